"""Tiny-size brute force, written independently of attn_oracle.c.

TEST INFRASTRUCTURE ONLY.

It materialises every per-pair score term as a [S, S, D/2] array, using an
explicit 2x2 rotation matrix R(phi) = [[cos, -sin], [sin, cos]] per pair
(the RoFormer rotation that "AttnFuse", section 2 "Rotary Position
Embeddings", refers to; NeoX pairing (r, r + D/2) per section 4.1), applies
the per-pair window of "ATFlash -- Per-RoPE-Wavelength Attention Windows"
("The idea") term by term, the causal mask, then softmax and PV with numpy.
Only meant for S, D of a few dozen.
"""
from __future__ import annotations

import numpy as np


def _rot(phi):
    c, s = np.cos(phi), np.sin(phi)
    return np.array([[c, -s], [s, c]])


def rotate(x: np.ndarray, theta: float, positions: np.ndarray) -> np.ndarray:
    """x: [S, D] fp64 -> rotated copy (pairs (r, r+D/2))."""
    S, D = x.shape
    h = D // 2
    out = x.copy()
    if theta == 0:
        return out
    for i, p in enumerate(positions):
        for r in range(h):
            ang = float(p) * theta ** (-2.0 * r / D)
            v = _rot(ang) @ np.array([x[i, r], x[i, r + h]])
            out[i, r], out[i, r + h] = v[0], v[1]
    return out


def pair_terms(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """[S, D] x [S, D] -> [S(query), S(key), D/2] per-pair products."""
    h = q.shape[1] // 2
    return (q[:, None, :h] * k[None, :, :h]) + (q[:, None, h:] * k[None, :, h:])


def attention_head(q, k, v, theta, causal, scale, window=None, pos_offset=0):
    """One head, fp64 inputs [S, D]; returns (out [S, D], scores [S, S])."""
    S, D = q.shape
    pos = np.arange(S) + pos_offset
    qr, kr = rotate(q, theta, pos), rotate(k, theta, pos)
    terms = pair_terms(qr, kr)
    if window is not None:
        dist = np.arange(S)[:, None] - np.arange(S)[None, :]
        keep = dist[:, :, None] <= np.asarray(window)[None, None, :]
        terms = np.where(keep, terms, 0.0)
    scores = scale * terms.sum(axis=2)
    if causal:
        scores = np.where(np.tril(np.ones((S, S), dtype=bool)), scores, -np.inf)
    mx = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - mx)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v, scores


def attention(q, k, v, theta, causal, scale, window=None, pos_offset=0):
    """[B, S, H, D] fp64 tensors (GQA by head grouping) -> [B, S, Hq, D]."""
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            o, _ = attention_head(q[b, :, h], k[b, :, h // g], v[b, :, h // g],
                                  theta, causal, scale, window, pos_offset)
            out[b, :, h] = o
    return out


def pruned_terms_count(window, S) -> int:
    """Count pruned (cell, pair) terms over the causal triangle one by one."""
    total = 0
    for n in range(S):
        for m in range(n + 1):
            for w in window:
                if n - m > w:
                    total += 1
    return total
