"""attn_decode_noalloc (through the C ABI) against attn_decode and the oracle.

The no-allocation entry point runs attn_decode's kernels with the split
partials in the library's static device scratch instead of a caller
workspace.  Two calls in a row, the second smaller, must each return
attn_decode's o and lse bit for bit and meet the oracle's bar (max |err| <=
2e-2, mean |err| <= 2e-3); a call that needs more than the scratch is
rejected before anything is launched.
"""
import math

import numpy as np
import pytest
import torch

from attention_attn_fwd_04_amd import binding
from attention_attn_fwd_04_amd.inputs import bf16_bits, make_qkv
from oracle import oracle as O

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 2e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _case(B, Hq, Hkv, L, D, theta, wk, num_splits, seed):
    # the cache from one seeded draw, the new query (position L-1) from another
    _, k, v = make_qkv(B, L, Hkv, Hkv, D, seed=seed)
    q = make_qkv(B, 1, Hq, Hkv, D, seed=seed + 1)[0][:, 0].contiguous()
    scale = 1 / math.sqrt(D)
    window = O.window_table(theta, D, wk) if wk else None
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o_ref, lse_ref = binding.attn_decode(qd, kd, vd, rope_theta=theta, scale=scale, window_table=window,
                                         num_splits=num_splits, want_lse=True)
    o = torch.empty_like(qd)
    lse = torch.empty(B, Hq, dtype=torch.float32, device="cuda:0")
    binding.attn_decode_noalloc(qd, kd, vd, o, lse, rope_theta=theta, scale=scale, window_table=window,
                                num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, lse_ref)
    ref, ref_lse = O.decode(bf16_bits(q), bf16_bits(k), bf16_bits(v), theta, scale, window, want_lse=True)
    for name, got, r in (("o", o.float().cpu().numpy(), ref), ("lse", lse.cpu().numpy(), ref_lse)):
        e = np.abs(got.astype(np.float64) - r)
        print("noalloc %s %s max_abs=%.3e mean_abs=%.3e" % ((B, Hq, Hkv, L, D, theta, wk, num_splits), name,
                                                              e.max(), e.mean()), flush=True)
        assert e.max() <= MAX_TOL and e.mean() <= MEAN_TOL


def test_noalloc_decode_two_calls_second_smaller():
    # a large call whose partials fill half the scratch (17 MiB), then a
    # smaller one: the second must not see the first's partials
    assert binding.attn_decode_workspace_bytes(4, 64, 8, 16384, 128, 128) > 16 << 20
    _case(4, 64, 8, 16384, 128, 5e5, None, 128, seed=11)
    _case(1, 8, 2, 300, 64, 1e4, 2.0, 7, seed=12)


def test_noalloc_decode_matches_with_window_and_gqa():
    _case(2, 16, 4, 3000, 128, 5e5, 2.0, 0, seed=13)
    _case(3, 12, 12, 77, 64, 0.0, None, 0, seed=14)


def test_noalloc_decode_rejects_beyond_scratch():
    B, Hq, Hkv, L, D = 64, 64, 8, 2048, 128
    k = torch.zeros(B, L, Hkv, D, dtype=torch.bfloat16, device="cuda:0")
    q = torch.zeros(B, Hq, D, dtype=torch.bfloat16, device="cuda:0")
    o = torch.empty_like(q)
    assert binding.attn_decode_workspace_bytes(B, Hq, Hkv, L, D, 64) > binding.attn_decode_scratch_bytes()
    with pytest.raises(binding.AttnError) as e:
        binding.attn_decode_noalloc(q, k, k, o, num_splits=64)
    assert e.value.status == binding.ATTN_ESCRATCH
    torch.cuda.synchronize()
