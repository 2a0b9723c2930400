"""Race check of the direct-to-LDS pipelines (GPU).

The library's kernels stream K, V (and cos/sin, Q, dO) tiles into LDS rings
with asynchronous direct loads and wait for them only where the schedule
needs them.  Its debug twin, libattn_mi355x_serial.so, is the same source
built with ATTN_SERIAL_LOADS=1: every such load is waited for in the same
instruction sequence that issues it, so no load is in flight while the
kernel goes on.  The arithmetic and its order are the same, so every output
must be bitwise equal between the two builds; a read of a slot whose load
the pipelined kernel had not waited for, or a load overwriting a slot that
another wave still reads, would make them differ.  Cases cover every entry
point that uses those pipelines (forward in all its variants, decode,
backward), ragged lengths, both head dimensions, GQA, the window and the
non-causal path.
"""
import math

import pytest
import torch

from attention_attn_fwd_04_amd import binding
from attention_attn_fwd_04_amd.inputs import make_qkv
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _both(fn):
    a = fn()
    torch.cuda.synchronize()
    with binding.use_library(binding.SERIAL_LIB_PATH):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    if isinstance(a, (tuple, list)):
        for i, (x, y) in enumerate(zip(a, b)):
            _same(x, y, "%s[%d]" % (what, i))
        return
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a, b), "%s: the serial-load build differs (max |diff| %s)" % (
        what, (a.float() - b.float()).abs().max().item())


def _gpu(*ts):
    return [t.to("cuda:0") for t in ts]


FWD_CASES = [
    # B, Hq, Hkv, S, D, theta, causal, window k
    (2, 4, 2, 700, 128, 1e4, True, None),      # ragged, GQA 2:1
    (1, 3, 1, 300, 64, 1e4, True, None),       # D = 64, GQA 3:1
    (1, 2, 2, 300, 128, 1e4, False, None),     # no causal mask
    (1, 4, 4, 1024, 128, 0.0, True, None),     # plain kernel (keys arrive rotated)
    (1, 2, 2, 2048, 128, 1e4, True, None),     # many tiles per wave
    (1, 4, 2, 700, 128, 5e5, True, 2.0),       # per-pair window
    (1, 2, 1, 600, 64, 1e4, True, 0.5),        # window, D = 64
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,theta,causal,wk", FWD_CASES)
def test_forward_serial_loads_bitwise(B, Hq, Hkv, S, D, theta, causal, wk):
    q, k, v = _gpu(*make_qkv(B, S, Hq, Hkv, D, seed=7000 + S + D))
    scale = 1 / math.sqrt(D)
    w = O.window_table(theta, D, wk) if wk else None
    kw = dict(rope_theta=theta, causal=causal, scale=scale, window_table=w)
    _same(*_both(lambda: binding.attn_fwd(q, k, v, **kw)), "attn_fwd")
    _same(*_both(lambda: binding.attn_fwd_lse(q, k, v, **kw)), "attn_fwd_lse")
    if causal and wk is None:
        _same(*_both(lambda: binding.attn_fwd_persistent(q, k, v, **kw)), "attn_fwd_persistent")
    if theta > 0:
        def rotated_k():
            _, kr = binding.attn_rope_apply(None, k, rope_theta=theta)
            return binding.attn_fwd_rotated_k(q, kr, v, **kw)
        _same(*_both(rotated_k), "attn_fwd_rotated_k")


@pytest.mark.parametrize("B,L,Hq,Hkv,D,theta,wk,ns", [
    (1, 5000, 16, 2, 128, 5e5, None, 0),
    (2, 3000, 8, 1, 64, 1e4, None, 7),
    (1, 5000, 16, 2, 128, 5e5, 2.0, 0),
])
def test_decode_serial_loads_bitwise(B, L, Hq, Hkv, D, theta, wk, ns):
    g = torch.Generator().manual_seed(7100 + L)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(B, L, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, L, Hkv, D, generator=g).to(torch.bfloat16)
    q, k, v = _gpu(q, k, v)
    w = O.window_table(theta, D, wk) if wk else None
    fn = lambda: binding.attn_decode(q, k, v, rope_theta=theta, scale=1 / math.sqrt(D), window_table=w,
                                     num_splits=ns, want_lse=True)
    _same(*_both(fn), "attn_decode")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,theta", [(1, 2, 2, 700, 128, 1e4), (1, 4, 2, 300, 64, 1e4)])
def test_backward_serial_loads_bitwise(B, Hq, Hkv, S, D, theta):
    q, k, v = _gpu(*make_qkv(B, S, Hq, Hkv, D, seed=7200 + S))
    scale = 1 / math.sqrt(D)
    dout = torch.randn(B, S, Hq, D, generator=torch.Generator().manual_seed(7300 + S)).to(torch.bfloat16).to("cuda:0")
    o, lse = binding.attn_fwd_lse(q, k, v, rope_theta=theta, causal=True, scale=scale)
    fn = lambda: binding.attn_bwd(q, k, v, o, lse, dout, rope_theta=theta, causal=True, scale=scale)
    _same(*_both(fn), "attn_bwd")
