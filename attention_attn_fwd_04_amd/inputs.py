"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

Holds none of the attention arithmetic: it only draws random numbers.
Recipe: a CPU torch.Generator seeded with `seed` draws fp32 Q, then K, then
V in [B, S, H, D] order; each is cast to bf16 with round-to-nearest-even.
dist="normal" draws N(0, 1) for all three; dist="uniform" draws Q, K from
U[-2, 2] and V from U[-1, 1].
"""
from __future__ import annotations

import torch

# name -> (B, Hq, Hkv, S, D, rope_theta, window_k_turns or None)
CONFIGS = {
    "tiny": dict(B=1, Hq=2, Hkv=2, S=256, D=64, theta=1e4, window_k=None),
    "prefill_s4096": dict(B=4, Hq=32, Hkv=32, S=4096, D=128, theta=1e4, window_k=None),
    "prefill_s8192": dict(B=4, Hq=32, Hkv=32, S=8192, D=128, theta=1e4, window_k=None),
    "gqa_s16384": dict(B=1, Hq=32, Hkv=8, S=16384, D=128, theta=5e5, window_k=None),
    "window_s32768": dict(B=1, Hq=32, Hkv=32, S=32768, D=128, theta=5e5, window_k=2.0),
}
CONFIG_SEEDS = {name: 42 + i for i, name in enumerate(CONFIGS)}


def make_qkv(B, S, Hq, Hkv, D, seed, dist="normal"):
    """Return CPU bf16 tensors q [B,S,Hq,D], k, v [B,S,Hkv,D]."""
    g = torch.Generator().manual_seed(int(seed))
    shapes = [(B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D)]
    out = []
    for i, shp in enumerate(shapes):
        if dist == "normal":
            t = torch.randn(shp, generator=g, dtype=torch.float32)
        elif dist == "uniform":
            lim = 1.0 if i == 2 else 2.0
            t = (torch.rand(shp, generator=g, dtype=torch.float32) * 2.0 - 1.0) * lim
        else:
            raise ValueError(dist)
        out.append(t.to(torch.bfloat16))
    return tuple(out)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a contiguous CPU bf16 tensor (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")
