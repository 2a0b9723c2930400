"""GPU parity of the forward kernels' softmax rescale (through the C ABI).

The forward kernels rescale O and l only when a later key tile scores more
than 14 log2 units above the reference taken from the first 64-key tile
(partial row sums of P above 2^14), or more than 128 (exp2 overflows to
+inf, the non-finite trigger); see tests/rescale_inputs.py.  Each case
first shows on the CPU, from the oracle's fp64 score rows, that the inputs
cross the trigger it is meant to reach, then compares the GPU output with
the oracle at the usual bar (max |err| <= 2e-2, mean |err| <= 2e-3) on
every path that shares the rescale: attn_fwd (fused RoPE and RoPE off),
the per-pair window, attn_fwd_lse (LSE against the oracle, o bitwise
attn_fwd's) and attn_fwd_persistent (bitwise attn_fwd's).  The online
softmax recurrence is exact ("AttnFuse", section 2), so the oracle's plain
softmax over the materialised row is the reference.
"""
import math

import numpy as np
import pytest
import torch

from attention_attn_fwd_04_amd import binding
from attention_attn_fwd_04_amd.inputs import CONFIGS, CONFIG_SEEDS, bf16_bits
from oracle import oracle as O
from rescale_inputs import FIRST_TILE, LAZY_LOG2, OVERFLOW_LOG2, make_rescale_qkv, score_gaps

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 2e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


# beta per head dimension: the moderate trigger (partial sums above 2^14) and
# the overflow trigger (scores more than 128 log2 units above the reference).
BETA = {("sum", 128): 5.0, ("sum", 64): 6.0, ("inf", 128): 20.0, ("inf", 64): 28.0}


def _inputs(B, S, Hq, Hkv, D, theta, kind, seed):
    return make_rescale_qkv(B, S, Hq, Hkv, D, theta, seed, alpha=1.0, beta=BETA[(kind, D)])


def _gap_rows(B, S, Hq, seed, n=12):
    rng = np.random.default_rng(seed)
    rows = [(0, FIRST_TILE, 0), (B - 1, S - 1, Hq - 1)]
    rows += [(int(rng.integers(B)), int(rng.integers(FIRST_TILE, S)), int(rng.integers(Hq))) for _ in range(n)]
    return np.array(rows, dtype=np.int32)


def _assert_trigger(q, k, theta, causal, scale, window, kind, rows):
    g = score_gaps(O, bf16_bits(q), bf16_bits(k), rows, theta, causal, scale, window)
    print("%s trigger: late-minus-first-tile gap (log2) min %.1f max %.1f" % (kind, g.min(), g.max()), flush=True)
    # every sampled row crosses the 2^14 trigger; the overflow case has rows
    # far past exp2's range
    assert g.min() > LAZY_LOG2 + 2.0, g.min()
    if kind == "inf":
        assert g.max() > OVERFLOW_LOG2 + 8.0, g.max()


def _err(o, ref, rows=None):
    got = o.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = np.stack([got[b, n, h] for b, n, h in rows])
    e = np.abs(got - ref)
    return float(e.max()), float(e.mean())


def _assert_bar(label, mx, mean):
    print("%s max_abs=%.3e mean_abs=%.3e" % (label, mx, mean), flush=True)
    assert mx <= MAX_TOL and mean <= MEAN_TOL, (label, mx, mean)


CASES = [
    # B, Hq, Hkv, S, D, theta, causal, window k, trigger
    (1, 4, 2, 700, 128, 1e4, True, None, "sum"),     # fused RoPE, ragged, GQA 2:1
    (1, 4, 2, 700, 128, 1e4, True, None, "inf"),
    (1, 3, 1, 300, 64, 1e4, True, None, "sum"),      # D = 64, GQA 3:1
    (1, 3, 1, 300, 64, 1e4, True, None, "inf"),
    (2, 2, 2, 520, 128, 0.0, True, None, "sum"),     # RoPE off
    (1, 2, 2, 300, 128, 1e4, False, None, "inf"),    # no causal mask
    (1, 4, 2, 700, 128, 5e5, True, 2.0, "sum"),      # per-pair window
    (1, 4, 2, 700, 128, 5e5, True, 2.0, "inf"),
    (1, 2, 2, 300, 64, 1e4, True, 2.0, "inf"),       # window, D = 64
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,theta,causal,wk,kind", CASES)
def test_rescale_fwd_lse_match_oracle(B, Hq, Hkv, S, D, theta, causal, wk, kind):
    label = "rescale %s" % ((B, Hq, Hkv, S, D, theta, causal, wk, kind),)
    print(label, flush=True)
    q, k, v = _inputs(B, S, Hq, Hkv, D, theta, kind, seed=6000 + S + D)
    scale = 1 / math.sqrt(D)
    window = O.window_table(theta, D, wk) if wk else None
    _assert_trigger(q, k, theta, causal, scale, window, kind, _gap_rows(B, S, Hq, seed=S))
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o = binding.attn_fwd(qd, kd, vd, rope_theta=theta, causal=causal, scale=scale, window_table=window)
    o2, lse = binding.attn_fwd_lse(qd, kd, vd, rope_theta=theta, causal=causal, scale=scale, window_table=window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    rows = O.all_rows(B, S, Hq)
    ref, ref_lse = O.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, theta, causal, scale, window,
                               want_lse=True)
    _assert_bar(label + " o", *_err(o, ref, rows))
    gl = lse.cpu().numpy().astype(np.float64)
    el = np.abs(np.array([gl[b, h, n] for b, n, h in rows]) - ref_lse)
    _assert_bar(label + " lse", float(el.max()), float(el.mean()))
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("D,kind", [(128, "sum"), (128, "inf"), (64, "inf")])
def test_rescale_persistent_bitwise_and_oracle(D, kind):
    """The persistent schedule runs the same per-tile code, rescale included:
    bitwise attn_fwd's output, and the oracle's to the bar."""
    B, Hq, Hkv, S, theta = 2, 4, 2, 700, 1e4
    q, k, v = _inputs(B, S, Hq, Hkv, D, theta, kind, seed=6100 + D)
    scale = 1 / math.sqrt(D)
    _assert_trigger(q, k, theta, True, scale, None, kind, _gap_rows(B, S, Hq, seed=D))
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o_p = binding.attn_fwd_persistent(qd, kd, vd, rope_theta=theta, causal=True, scale=scale)
    o_r = binding.attn_fwd(qd, kd, vd, rope_theta=theta, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p.view(torch.int16), o_r.view(torch.int16))
    ref = O.attn_full(bf16_bits(q), bf16_bits(k), bf16_bits(v), theta, True, scale, None)
    _assert_bar("persistent rescale D=%d %s" % (D, kind), *_err(o_p, ref))


def _sample_rows(B, S, Hq, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(6):
        b, h = int(rng.integers(B)), int(rng.integers(Hq))
        picks = {0, 1, 63, 64, 65, 255, 256, S // 2, S - 257, S - 2, S - 1}
        picks |= set(int(x) for x in rng.integers(FIRST_TILE, S, 4))
        rows += [(b, n, h) for n in sorted(p for p in picks if 0 <= p < S)]
    return np.array(rows, dtype=np.int32)


@pytest.mark.parametrize("name,kind", [("prefill_s8192", "sum"), ("prefill_s8192", "inf"), ("window_s32768", "sum")])
def test_rescale_full_size_sampled(name, kind):
    """The full configurations in the benchmark's launch configuration, on
    sampled rows: attn_fwd (fused RoPE; the window at window_s32768),
    attn_fwd_lse, and at prefill_s8192 attn_fwd_persistent bitwise."""
    cfg = CONFIGS[name]
    B, Hq, Hkv, S, D, theta = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["S"], cfg["D"], cfg["theta"]
    print("rescale full size %s %s" % (name, kind), flush=True)
    window = O.window_table(theta, D, cfg["window_k"]) if cfg["window_k"] else None
    q, k, v = _inputs(B, S, Hq, Hkv, D, theta, kind, seed=CONFIG_SEEDS[name] + 700)
    scale = 1 / math.sqrt(D)
    rows = _sample_rows(B, S, Hq, seed=CONFIG_SEEDS[name])
    late = rows[rows[:, 1] >= FIRST_TILE]
    _assert_trigger(q, k, theta, True, scale, window, kind, late[::4])
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = binding.attn_fwd_lse(qd, kd, vd, rope_theta=theta, causal=True, scale=scale, window_table=window)
    o_r = binding.attn_fwd(qd, kd, vd, rope_theta=theta, causal=True, scale=scale, window_table=window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_r.view(torch.int16))
    if window is None:
        o_p = binding.attn_fwd_persistent(qd, kd, vd, rope_theta=theta, causal=True, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o_p.view(torch.int16), o_r.view(torch.int16))
        del o_p
    ref, ref_lse = O.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, theta, True, scale, window,
                               want_lse=True)
    _assert_bar("rescale %s %s o" % (name, kind), *_err(o, ref, rows))
    gl = lse.cpu().numpy().astype(np.float64)
    el = np.abs(np.array([gl[b, h, n] for b, n, h in rows]) - ref_lse)
    _assert_bar("rescale %s %s lse" % (name, kind), float(el.max()), float(el.mean()))
    assert torch.isfinite(o.float()).all()
