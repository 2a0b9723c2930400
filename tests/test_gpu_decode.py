"""GPU parity of attn_decode (split-KV decode, through the C ABI) against the
fp64 oracle's decode.

Bar: max |err| <= 2e-2 and mean |err| <= 2e-3 over the outputs, and the same
for the natural-log LSE (its error is that of the scaled scores: bf16 Q' and
bf16 P, as for attn_fwd_lse).  The cache keys are used as stored, so the
oracle gets the same bits; one end-to-end case builds the cache with
attn_rope_apply and compares with the prefill oracle's last row instead.
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


def _inputs(B, L, Hq, Hkv, D, seed):
    q, k, v = make_qkv(B, L, Hq, Hkv, D, seed)
    return q[:, -1].contiguous(), k, v          # the newest token's queries, the cache


def _check(name, got, ref):
    err = np.abs(got.astype(np.float64) - ref)
    print("%s max_abs=%.3e mean_abs=%.3e" % (name, err.max(), err.mean()), flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_TOL and err.mean() <= MEAN_TOL, (name, err.max(), err.mean())


CASES = [
    # B, L, Hq, Hkv, D, theta, window k, num_splits
    (1, 1, 8, 2, 128, 1e4, None, 0),           # a single cached key
    (2, 31, 8, 8, 64, 1e4, None, 0),           # one partial tile, no GQA
    (1, 1000, 64, 8, 128, 5e5, None, 0),       # Llama-3-70B heads, ragged length
    (3, 777, 32, 8, 128, 0.0, None, 0),        # RoPE off, B = 3
    (1, 4096, 32, 4, 128, 1e4, None, 1),       # unsplit
    (1, 4096, 32, 4, 128, 1e4, None, 128),     # one tile per split
    (1, 3000, 8, 1, 64, 1e4, None, 7),         # 8 heads on one KV head, uneven splits
    (1, 100, 32, 1, 128, 1e4, None, 0),        # 32 query heads per KV head (all MFMA columns)
    (1, 5000, 16, 2, 128, 5e5, 2.0, 0),        # per-pair window
    (1, 600, 4, 2, 64, 1e4, 0.5, 0),           # window, D = 64, partial pairs at short range
]


@pytest.mark.parametrize("B,L,Hq,Hkv,D,theta,wk,ns", CASES)
def test_decode_matches_oracle(B, L, Hq, Hkv, D, theta, wk, ns):
    q, k, v = _inputs(B, L, Hq, Hkv, D, seed=5000 + L + D)
    scale = 1 / math.sqrt(D)
    window = O.window_table(theta if theta else 1e4, D, wk) if wk else None
    o, lse = binding.attn_decode(q.cuda(), k.cuda(), v.cuda(), rope_theta=theta, scale=scale,
                                 window_table=window, num_splits=ns, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.decode(bf16_bits(q), bf16_bits(k), bf16_bits(v), theta, scale, window, want_lse=True)
    label = "decode %s" % ((B, L, Hq, Hkv, D, theta, wk, ns),)
    _check(label, o.float().cpu().numpy(), ref)
    _check(label + " lse", lse.cpu().numpy(), ref_lse)


def test_decode_split_count_does_not_change_the_result_beyond_rounding():
    q, k, v = _inputs(1, 2500, 16, 4, 128, seed=91)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    outs = [binding.attn_decode(qd, kd, vd, rope_theta=1e4, num_splits=n).float().cpu().numpy()
            for n in (1, 3, 0, 79)]
    for x in outs[1:]:
        assert np.abs(x - outs[0]).max() <= 1e-2


def test_decode_with_cache_from_rope_pass_matches_prefill_row():
    """End to end: K cache rotated by attn_rope_apply; the reference is the
    prefill oracle's row L-1 on the raw inputs (RoPE on q and k in fp64)."""
    B, L, Hq, Hkv, D, theta = 1, 700, 16, 4, 128, 1e4
    q, k, v = make_qkv(B, L, Hq, Hkv, D, seed=92)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    _, kr = binding.attn_rope_apply(qd, kd, rope_theta=theta)
    o = binding.attn_decode(qd[:, -1].contiguous(), kr, vd, rope_theta=theta)
    torch.cuda.synchronize()
    rows = np.array([(0, L - 1, h) for h in range(Hq)], dtype=np.int32)
    ref = O.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, theta, True, 1 / math.sqrt(D))
    _check("decode end-to-end", o.float().cpu().numpy()[0], ref)


def test_decode_full_size_llama70b_32k():
    """Llama-3-70B attention shape (64 query heads, 8 KV heads, D = 128) at a
    32k cache: every head against the oracle."""
    B, L, Hq, Hkv, D, theta = 1, 32768, 64, 8, 128, 5e5
    q, k, v = _inputs(B, L, Hq, Hkv, D, seed=93)
    o, lse = binding.attn_decode(q.cuda(), k.cuda(), v.cuda(), rope_theta=theta, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.decode(bf16_bits(q), bf16_bits(k), bf16_bits(v), theta, 1 / math.sqrt(D), want_lse=True)
    _check("decode 70B 32k", o.float().cpu().numpy(), ref)
    _check("decode 70B 32k lse", lse.cpu().numpy(), ref_lse)
