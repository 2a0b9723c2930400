"""The acceptance bar for bf16 gradients, shared by the backward GPU tests,
the fuzzer and the CPU controls that show the bar rejects plausible slips.

"AttnFuse", section 6.6 "Correctness", checks gradients against a plain
reference at FA2's |err| < 2e-2.  The gradients are stored in bf16, whose
round-to-nearest-even error is up to 2^-8 |g| (half an ulp of the 8-bit
significand), so the element bar is 2e-2 + 2^-8 |ref|: the absolute bar plus
one rounding of the stored value.

The mean bar is 2e-3 + 2^-8 mean|ref| per tensor.  Its relative term follows
the rounding chain of the kernels, not a single rounding: a gradient element
carries the error of its own bf16 store (mean about 2^-9.5 |g| for
round-to-nearest over uniformly spread significands) plus three upstream
roundings of the same size that enter its sum with random signs (the staged
query or rotated key, dS = P (dP - Delta) rounded to bf16 for the MFMA, and
Delta taken from the bf16 forward output), about 2 x 2^-9.5 = 2^-8.5 |g| in
all.  The CPU emulation of that chain in tests/test_bwd_bar_controls.py
measures it, and the same file shows that each plausible slip (a missing
inverse rotation, a missing scale, a neighbour's Delta, a dropped GQA
partial, ...) fails the bar by a wide margin.
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 2e-2
REL_TOL = 2.0 ** -8
MEAN_ABS_TOL = 2e-3
MEAN_REL_TOL = 2.0 ** -8


def grad_bar(got, ref):
    """(ok, details) for one gradient tensor against its fp64 reference."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bar = ABS_TOL + REL_TOL * np.abs(ref)
    finite = bool(np.isfinite(got).all())
    elem_ok = bool((err <= bar).all())
    mean_bar = MEAN_ABS_TOL + MEAN_REL_TOL * float(np.abs(ref).mean())
    mean_ok = err.size < 32 or float(err.mean()) <= mean_bar
    worst = np.unravel_index(int(np.argmax(err - bar)), err.shape)
    return finite and elem_ok and mean_ok, dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                                                 mean_bar=mean_bar, worst=worst, elem_ok=elem_ok, mean_ok=mean_ok,
                                                 finite=finite)
