"""GPU parity of attn_fwd_lse (through the C ABI) against the fp64 oracle.

The LSE of a row is a softmax-weighted mean of its scores plus log l, so its
error is that of the scores (the kernel rounds Q' and K' to bf16: a relative
2^-9 per element, about 4e-3 per scaled score for N(0,1) inputs at D = 128)
plus the relative error of l (an fp32 sum of probabilities computed from
those scores; the fp32 rounding of the sum adds well under 2^-9).  The same bar as the outputs therefore applies: max |err| <= 2e-2 and
mean |err| <= 2e-3.  o must be bitwise the output of attn_fwd.
"""
import math

import numpy as np
import pytest
import torch

from attention_attn_fwd_04_amd import binding
from attention_attn_fwd_04_amd.inputs import CONFIGS, CONFIG_SEEDS, bf16_bits, make_qkv
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


def _check(lse_dev, q, k, v, rows, theta, causal, scale, window, label):
    _, ref = O.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, theta, causal, scale, window,
                         want_lse=True)
    got = lse_dev.cpu().numpy().astype(np.float64)
    g = np.array([got[b, h, n] for b, n, h in rows])
    err = np.abs(g - ref)
    print("%s lse max_abs=%.3e mean_abs=%.3e" % (label, err.max(), err.mean()), flush=True)
    assert np.isfinite(g).all()
    assert err.max() <= MAX_TOL, (label, err.max())
    # The mean bar is a statistic over many rows (random rounding errors of
    # the scores average out); over a handful of rows it is the max bar.
    if err.size >= 32:
        assert err.mean() <= MEAN_TOL, (label, err.mean())


CASES = [
    # B, Hq, Hkv, S, D, theta, causal, window k
    (1, 2, 2, 256, 64, 1e4, True, None),
    (2, 4, 2, 700, 128, 1e4, True, None),     # ragged, GQA 2:1
    (1, 8, 2, 520, 128, 5e5, True, None),     # GQA 4:1
    (1, 2, 2, 300, 128, 1e4, False, None),    # no causal mask
    (1, 2, 2, 384, 128, 0.0, True, None),     # RoPE off
    (1, 1, 1, 1, 128, 1e4, True, None),       # single token: L = scale q0.k0
    (1, 2, 2, 1100, 128, 5e5, True, 0.25),    # window, partial pairs at short range
    (1, 2, 2, 600, 64, 1e4, True, 0.5),       # window, D = 64
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,theta,causal,wk", CASES)
def test_lse_matches_oracle_and_o_is_unchanged(B, Hq, Hkv, S, D, theta, causal, wk):
    q, k, v = make_qkv(B, S, Hq, Hkv, D, seed=3000 + S + D)
    scale = 1 / math.sqrt(D)
    window = O.window_table(theta, D, wk) if wk else None
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o_ref = binding.attn_fwd(qd, kd, vd, rope_theta=theta, causal=causal, scale=scale, window_table=window)
    o, lse = binding.attn_fwd_lse(qd, kd, vd, rope_theta=theta, causal=causal, scale=scale, window_table=window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    rows = O.all_rows(B, S, Hq)
    _check(lse, q, k, v, rows, theta, causal, scale, window, "lse %s" % ((B, Hq, Hkv, S, D, theta, causal, wk),))


def test_lse_of_zero_queries_is_log_of_key_count():
    """Q = 0: every score is 0 and the causal row n sees n + 1 keys."""
    B, H, S, D = 1, 2, 600, 128
    _, k, v = make_qkv(B, S, H, H, D, seed=77)
    q = torch.zeros(B, S, H, D, dtype=torch.bfloat16)
    _, lse = binding.attn_fwd_lse(q.cuda(), k.cuda(), v.cuda(), rope_theta=1e4, causal=True)
    torch.cuda.synchronize()
    ref = np.log(np.arange(1, S + 1, dtype=np.float64))
    err = np.abs(lse.cpu().numpy().astype(np.float64) - ref[None, None, :]).max()
    assert err <= 1e-5 * math.log(S), err   # exact up to the fp32 log of a sum of ones


@pytest.mark.parametrize("name", ["prefill_s8192", "window_s32768"])
def test_lse_full_size_sampled(name):
    """At the full configuration, sampled rows: the first and last row of
    sampled query tiles, rows next to the diagonal, and random rows."""
    cfg = CONFIGS[name]
    B, Hq, Hkv, S, D, theta = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["theta"]
    window = O.window_table(theta, D, cfg["window_k"]) if cfg["window_k"] else None
    q, k, v = make_qkv(B, S, Hq, Hkv, D, seed=CONFIG_SEEDS[name])
    scale = 1 / math.sqrt(D)
    _, lse = binding.attn_fwd_lse(q.cuda(), k.cuda(), v.cuda(), rope_theta=theta, causal=True, scale=scale,
                                  window_table=window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = [(0, 0, 0), (B - 1, S - 1, Hq - 1), (0, 255, 1), (0, 256, 1), (B - 1, S // 2, 3)]
    rows += [(int(rng.integers(B)), int(rng.integers(S)), int(rng.integers(Hq))) for _ in range(11)]
    _check(lse, q, k, v, np.array(rows, dtype=np.int32), theta, True, scale, window, "lse %s" % name)
