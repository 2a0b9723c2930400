"""GPU parity of the persistent, cost-balanced schedule (attn_fwd_persistent,
"Croqtile", "Step 4"): the same per-tile computation as attn_fwd on a
host-built task list, so the outputs must match attn_fwd bit for bit, and
the fp64 oracle to the bf16 bar (max |err| <= 2e-2, mean <= 2e-3)."""
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


CASES = [
    # B, Hq, Hkv, S, D, theta: several tiles per bin, ragged tails, GQA, both D
    (1, 2, 2, 256, 64, 1e4),       # the tiny configuration: 2 tiles, 2 bins
    (2, 4, 2, 700, 128, 1e4),      # ragged, 8 heads: XCD groups
    (1, 8, 2, 520, 128, 5e5),      # GQA 4:1
    (1, 3, 1, 300, 64, 1e4),       # D = 64, 3 heads: one group
    (1, 2, 2, 384, 128, 0.0),      # RoPE off
    (1, 2, 1, 1, 128, 1e4),        # single token
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,theta", CASES)
def test_persistent_matches_oracle_and_attn_fwd(B, Hq, Hkv, S, D, theta):
    q, k, v = make_qkv(B, S, Hq, Hkv, D, seed=3000 + S + D)
    scale = 1 / math.sqrt(D)
    print("persistent case", (B, Hq, Hkv, S, D, theta), flush=True)
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    o_p = binding.attn_fwd_persistent(qd, kd, vd, rope_theta=theta, causal=True, scale=scale)
    o_r = binding.attn_fwd(qd, kd, vd, rope_theta=theta, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_r)
    ref = O.attn_full(bf16_bits(q), bf16_bits(k), bf16_bits(v), theta, True, scale, None)
    err = np.abs(o_p.cpu().float().numpy().astype(np.float64) - ref)
    print("max_abs=%.3e mean_abs=%.3e" % (err.max(), err.mean()), flush=True)
    assert err.max() <= MAX_TOL and err.mean() <= MEAN_TOL


def test_persistent_many_tiles_per_bin():
    """More tiles than compute units: B2 H16 S4096 = 512 tiles, two or more
    per bin, so consecutive tiles of one work-group reuse its LDS."""
    B, Hq, Hkv, S, D = 2, 16, 16, 4096, 128
    q, k, v = make_qkv(B, S, Hq, Hkv, D, seed=3101)
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    o_p = binding.attn_fwd_persistent(qd, kd, vd, rope_theta=1e4, causal=True)
    o_r = binding.attn_fwd(qd, kd, vd, rope_theta=1e4, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_r)
    rows = [(0, 0, 0), (1, 4095, 15), (0, 1000, 7), (1, 2047, 3), (0, 256, 12)]
    ref = O.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, 1e4, True, 1 / math.sqrt(D))
    got = o_p.cpu().float().numpy().astype(np.float64)
    err = np.abs(np.stack([got[b, n, h] for b, n, h in rows]) - ref)
    assert err.max() <= MAX_TOL and err.mean() <= MEAN_TOL


def test_persistent_noncausal_runs_regular_schedule():
    q, k, v = make_qkv(1, 300, 2, 2, 128, seed=3102)
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    o_p = binding.attn_fwd_persistent(qd, kd, vd, rope_theta=1e4, causal=False)
    o_r = binding.attn_fwd(qd, kd, vd, rope_theta=1e4, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_r)


def test_persistent_rejects_window():
    q, k, v = make_qkv(1, 256, 2, 2, 128, seed=3103)
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    w = binding.attn_window_table(5e5, 128, 2.0)
    with pytest.raises(binding.AttnError) as e:
        binding.attn_fwd_persistent(qd, kd, vd, rope_theta=5e5, causal=True, window_table=w)
    assert e.value.status == binding.ATTN_EUNSUPPORTED


@pytest.mark.parametrize("name", ["prefill_s8192", "gqa_s16384"])
def test_persistent_full_size_bitwise(name):
    """At the measured sizes (one work-group per CU, 8-16 tiles each) the
    output equals attn_fwd's bit for bit, and sampled rows meet the oracle bar."""
    c = CONFIGS[name]
    B, Hq, Hkv, S, D, theta = c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], c["theta"]
    print("persistent full size", name, flush=True)
    q, k, v = make_qkv(B, S, Hq, Hkv, D, seed=CONFIG_SEEDS[name])
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    o_p = binding.attn_fwd_persistent(qd, kd, vd, rope_theta=theta, causal=True)
    o_r = binding.attn_fwd(qd, kd, vd, rope_theta=theta, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_r)
    rows = [(0, 0, 0), (B - 1, S - 1, Hq - 1), (0, S // 2 + 3, Hq // 2), (B - 1, 255, 1), (0, 256, Hq - 2)]
    ref = O.attn_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, theta, True, 1 / math.sqrt(D))
    got = o_p.cpu().float().numpy().astype(np.float64)
    err = np.abs(np.stack([got[b, n, h] for b, n, h in rows]) - ref)
    print("max_abs=%.3e mean_abs=%.3e" % (err.max(), err.mean()), flush=True)
    assert err.max() <= MAX_TOL and err.mean() <= MEAN_TOL
