"""CPU pins of the inputs the rescale GPU tests use (tests/rescale_inputs.py).

From the oracle's fp64 score rows: every query row past the first 64-key
tile scores more than 14 log2 units higher on some later key than anywhere
in the first tile (the forward kernels' lazy-rescale trigger, a partial row
sum of P above 2^14), and the overflow inputs put some rows more than 128
units higher (exp2 overflows in fp32, the non-finite trigger).  Rows inside
the first tile keep the N(0, 1) score scale.
"""
import math

import numpy as np
import pytest

from attention_attn_fwd_04_amd.inputs import bf16_bits, make_qkv
from oracle import oracle as O
from rescale_inputs import FIRST_TILE, LAZY_LOG2, LOG2E, OVERFLOW_LOG2, make_rescale_qkv, score_gaps


@pytest.mark.parametrize("S,D,theta,wk,beta,overflow", [
    (700, 128, 1e4, None, 5.0, False),
    (700, 128, 1e4, None, 20.0, True),
    (300, 64, 1e4, None, 6.0, False),
    (300, 64, 1e4, None, 28.0, True),
    (520, 128, 0.0, None, 5.0, False),
    (700, 128, 5e5, 2.0, 5.0, False),
    (700, 128, 5e5, 2.0, 20.0, True),
])
def test_rescale_inputs_cross_the_trigger(S, D, theta, wk, beta, overflow):
    B, Hq, Hkv = 1, 2, 1
    q, k, _ = make_rescale_qkv(B, S, Hq, Hkv, D, theta, seed=11 + S, alpha=1.0, beta=beta)
    scale = 1 / math.sqrt(D)
    window = O.window_table(theta, D, wk) if wk else None
    rows = np.array([(0, n, h) for n in range(FIRST_TILE, S, 7) for h in range(Hq)], dtype=np.int32)
    g = score_gaps(O, bf16_bits(q), bf16_bits(k), rows, theta, True, scale, window)
    assert g.min() > LAZY_LOG2 + 2.0, g.min()
    if overflow:
        assert g.max() > OVERFLOW_LOG2 + 8.0, g.max()
    else:
        assert g.max() < OVERFLOW_LOG2, g.max()


def test_first_tile_rows_keep_normal_scores():
    """Rows n < 64 have u's pairs zeroed, so the large -beta u of the early
    keys does not enter their scores: they match plain N(0, 1) rows in size."""
    S, D = 300, 128
    q, k, _ = make_rescale_qkv(1, S, 2, 1, D, 1e4, seed=5, alpha=1.0, beta=20.0)
    qn, kn, _ = make_qkv(1, S, 2, 1, D, seed=5)
    scale = 1 / math.sqrt(D)
    for n in (0, 17, 63):
        s = O.scores_row(bf16_bits(q), bf16_bits(k), 0, n, 0, 1e4, True, scale)[:n + 1] * LOG2E
        s0 = O.scores_row(bf16_bits(qn), bf16_bits(kn), 0, n, 0, 1e4, True, scale)[:n + 1] * LOG2E
        assert np.abs(s).max() < 4.0 * max(1.0, np.abs(s0).max())
