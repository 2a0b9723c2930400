"""Inputs that force the forward kernels' rare softmax rescale.

Online softmax ("Flash Attention: Causal Prefill D=128", "Online softmax:
what must remain invariant"; "AttnFuse", section 2) keeps a running max and
rescales O and l by alpha = exp2(m_old - m_new) when a later key tile scores
above it.  The forward kernel takes that step lazily: P is computed against a
reference m_ref, the row max of the first 64-key tile, and only when a lane's
partial row sum of P over a tile exceeds 2^14 (one score more than 14 log2
units above m_ref suffices), or is not finite (a score more than 128 log2
units above it: exp2 overflows), does the tile raise m_ref and rescale.
N(0, 1) inputs never get there (gaps of a few units), so these inputs make
the first tile score far below the later ones for every query row n >= 64:

  * a fixed sign vector u on `u_pairs` of the D/2 rotation pairs (the
    lowest-frequency ones), zero on the others;
  * q_n = g_n + alpha R(n)^T u for n >= 64, and for n < 64 g_n with u's pairs
    zeroed (so those rows, which see only the first tile, keep N(0,1)-sized
    scores and need no rescale);
  * k_m = g'_m - beta R(m)^T u for the first-tile keys m < 64, k_m = g'_m
    after them.

R(p) is the RoPE rotation of position p (NeoX pairs (r, r + D/2), angle
p theta^(-2r/D), "AttnFuse", section 2), so after the kernels rotate q and k
the query carries +alpha u and the early keys -beta u: the early scores drop
by about alpha beta |u|^2 scale (natural units), while the later keys'
scores stay of N(0, 1) size.  The early keys then weigh 2^-gap in the
softmax, so their large magnitudes cost no accuracy.  g, g', v are the
seeded N(0, 1) draws of `make_qkv`.  The construction only shapes inputs;
what the tests compare against is the oracle on the resulting bf16 bits,
and the gap itself is read from the oracle's score rows (`score_gaps`).
"""
from __future__ import annotations

import numpy as np
import torch

from attention_attn_fwd_04_amd.inputs import make_qkv

LOG2E = 1.4426950408889634
FIRST_TILE = 64          # keys in the forward kernel's first (reference) tile
LAZY_LOG2 = 14.0         # a partial row sum of P above 2^14 triggers the rescale
OVERFLOW_LOG2 = 128.0    # exp2 of more than 128 is +inf in fp32


def _u_vector(D, u_pairs, seed):
    rng = np.random.default_rng(seed)
    h = D // 2
    sel = np.arange(h - u_pairs, h)
    u = np.zeros(D)
    u[sel] = rng.choice([-1.0, 1.0], size=u_pairs)
    u[sel + h] = rng.choice([-1.0, 1.0], size=u_pairs)
    return u, sel


def _inv_rotated_rows(S, D, theta, u):
    """Rows R(p)^T u for p = 0 .. S-1 (fp64)."""
    out = np.tile(u, (S, 1))
    if theta == 0.0:
        return out
    h = D // 2
    inv = theta ** (-2.0 * np.arange(h) / D)
    ang = np.arange(S, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x, y = u[None, :h], u[None, h:]
    out[:, :h] = c * x + s * y
    out[:, h:] = -s * x + c * y
    return out


def make_rescale_qkv(B, S, Hq, Hkv, D, theta, seed, alpha=1.0, beta=4.0, u_pairs=None):
    """bf16 CPU tensors q [B,S,Hq,D], k, v [B,S,Hkv,D] built as described above."""
    if u_pairs is None:
        u_pairs = D // 4
    q, k, v = make_qkv(B, S, Hq, Hkv, D, seed=seed)
    u, sel = _u_vector(D, u_pairs, seed)
    t = torch.from_numpy(_inv_rotated_rows(S, D, theta, u)).float()
    qf, kf = q.float(), k.float()
    n0 = min(S, FIRST_TILE)
    if S > FIRST_TILE:
        qf[:, FIRST_TILE:] += alpha * t[None, FIRST_TILE:, None, :]
    keep = torch.ones(D)
    keep[torch.from_numpy(sel)] = 0.0
    keep[torch.from_numpy(sel + D // 2)] = 0.0
    qf[:, :n0] *= keep
    kf[:, :n0] -= beta * t[None, :n0, None, :]
    return qf.to(torch.bfloat16), kf.to(torch.bfloat16), v


def score_gaps(oracle, q_bits, k_bits, rows, theta, causal, scale, window=None):
    """For each query row (b, n, hq): the largest scaled score (log2 units)
    among the keys after the first tile minus the largest within it, from
    the oracle's fp64 score rows."""
    out = []
    for b, n, h in rows:
        s = oracle.scores_row(q_bits, k_bits, int(b), int(n), int(h), theta, causal, scale, window) * LOG2E
        first = np.max(s[:FIRST_TILE])
        later = s[FIRST_TILE:]
        later = later[np.isfinite(later)]
        out.append((later.max() if later.size else -np.inf) - first)
    return np.array(out)
