"""Host-side checks of the C-ABI library (CPU only, no device work).

The library must load, export every function include/attn.h declares, and
its host-only helpers must agree bit for bit with the oracle's independent
implementations.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from attention_attn_fwd_04_amd import binding
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "attn.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding.LIB_PATH)
    names = _declared_functions()
    assert "attn_fwd" in names and "attn_rope_apply" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(binding.EXPORTED) == set(names)


def test_serial_load_build_exports_the_same_symbols():
    """The debug twin (every direct-to-LDS load waited for as it is issued),
    which the GPU race check compares against, is built beside the library
    and exports the same C ABI."""
    lib = ctypes.CDLL(binding.SERIAL_LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_use_library_routes_calls_and_restores():
    """binding.use_library switches the wrappers to another build inside the
    block (host-only calls here) and back to the library afterwards."""
    main = binding.lib()
    with binding.use_library(binding.SERIAL_LIB_PATH) as serial:
        assert binding.lib() is serial and serial is not main
        assert binding.strerror(binding.ATTN_EINVAL) == main.attn_strerror(binding.ATTN_EINVAL).decode()
    assert binding.lib() is main
    try:
        with binding.use_library(binding.SERIAL_LIB_PATH):
            raise KeyError("inside")
    except KeyError:
        pass
    assert binding.lib() is main


def test_strerror_covers_every_status():
    for st in range(0, -8, -1):
        msg = binding.strerror(st)
        assert msg and msg != "unknown status"
    assert binding.strerror(-99) == "unknown status"


@pytest.mark.parametrize("theta,D,k", [(5e5, 128, 2.0), (1e4, 64, 2.0), (1e4, 128, 2.0),
                                       (5e5, 128, 1.0), (1e6, 128, 3.0)])
def test_window_table_bit_exact_vs_oracle(theta, D, k):
    np.testing.assert_array_equal(binding.attn_window_table(theta, D, k), O.window_table(theta, D, k))


@pytest.mark.parametrize("S", [0, 1, 2, 13, 256, 4096, 8192, 16384, 32768, 1 << 20])
def test_pruned_terms_bit_exact_vs_oracle(S):
    for theta, D in ((5e5, 128), (1e4, 64), (1e4, 128)):
        w = O.window_table(theta, D, 2.0)
        assert binding.attn_pruned_terms(w, D, S) == O.pruned_terms(w, D, S)
    rng = np.random.default_rng(S)
    w = np.sort(rng.integers(-3, max(S, 1) + 5, size=64)).astype(np.int32)
    assert binding.attn_pruned_terms(w, 128, S) == O.pruned_terms(w, 128, S)


def test_window_s32768_closed_form_value():
    """theta=5e5, D=128, k=2 at S=32768: 16,939,317,408 pruned pair terms per head,
    49.3 % of the 64 * S(S+1)/2 pair terms (closed form, independent of input)."""
    w = binding.attn_window_table(5e5, 128, 2.0)
    per_head = binding.attn_pruned_terms(w, 128, 32768)
    assert per_head == O.pruned_terms(O.window_table(5e5, 128, 2.0), 128, 32768)
    assert abs(per_head / (64 * 32768 * 32769 / 2) - 0.4930) < 5e-4


A = 1 << 20  # fake, 16-byte aligned addresses: attn_check_args never dereferences them


def _chk(**kw):
    args = dict(q=A, k=A * 64, v=A * 128, o=A * 192, B=1, Hq=4, Hkv=2, S=128, D=128,
                rope_theta=1e4, causal=1, scale=0.088, window_table=None)
    args.update(kw)
    return binding.attn_check_args(args["q"], args["k"], args["v"], args["o"], args["B"], args["Hq"],
                                   args["Hkv"], args["S"], args["D"], args["rope_theta"], args["causal"],
                                   args["scale"], args["window_table"])


def test_check_args_accepts_valid():
    assert _chk() == binding.ATTN_OK
    assert _chk(rope_theta=0.0) == binding.ATTN_OK
    assert _chk(D=64, Hq=8, Hkv=1) == binding.ATTN_OK
    assert _chk(S=0) == binding.ATTN_OK and _chk(B=0) == binding.ATTN_OK
    assert _chk(S=0, q=0, k=0, v=0, o=0) == binding.ATTN_OK  # empty tensors may have NULL data
    assert _chk(causal=0) == binding.ATTN_OK
    assert _chk(window_table=O.window_table(5e5, 128, 2.0)) == binding.ATTN_OK


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), binding.ATTN_EINVAL),
    (dict(q=0, S=16), binding.ATTN_EINVAL),
    (dict(o=0), binding.ATTN_EINVAL),
    (dict(q=A + 8), binding.ATTN_EALIGN),
    (dict(v=A * 128 + 2), binding.ATTN_EALIGN),
    (dict(D=96), binding.ATTN_EUNSUPPORTED),
    (dict(D=256), binding.ATTN_EUNSUPPORTED),
    (dict(D=7), binding.ATTN_EINVAL),
    (dict(Hq=3, Hkv=2), binding.ATTN_EINVAL),
    (dict(Hq=0), binding.ATTN_EINVAL),
    (dict(B=-1), binding.ATTN_EINVAL),
    (dict(S=-5), binding.ATTN_EINVAL),
    (dict(scale=0.0), binding.ATTN_EINVAL),
    (dict(scale=-1.0), binding.ATTN_EINVAL),
    (dict(scale=float("nan")), binding.ATTN_EINVAL),
    (dict(scale=float("inf")), binding.ATTN_EINVAL),
    (dict(rope_theta=float("nan")), binding.ATTN_EINVAL),
    (dict(rope_theta=0.5), binding.ATTN_EINVAL),
    (dict(rope_theta=-1e4), binding.ATTN_EINVAL),
    (dict(causal=2), binding.ATTN_EINVAL),
    (dict(o=A), binding.ATTN_EINVAL),                     # o aliases q
    (dict(o=A * 128 + 256), binding.ATTN_EINVAL),         # o overlaps v
    (dict(window_table=np.arange(64)[::-1].copy()), binding.ATTN_EINVAL),  # not monotone
    (dict(window_table=np.arange(64), causal=0), binding.ATTN_EINVAL),     # window needs causal
])
def test_check_args_rejects(kw, status):
    assert _chk(**kw) == status


def test_window_table_argument_errors():
    for args in ((1.0, 128, 2.0), (5e5, 127, 2.0), (5e5, 128, 0.0), (float("nan"), 128, 2.0)):
        with pytest.raises(binding.AttnError):
            binding.attn_window_table(*args)


def _lse_call(lse, S=128):
    """attn_fwd_lse with fake device addresses: only argument errors that are
    caught before any device call are exercised here."""
    return binding.lib().attn_fwd_lse(A, A * 64, A * 128, A * 192, lse, 1, 4, 2, S, 128,
                                      1e4, 1, 0.088, None, None)


@pytest.mark.parametrize("lse,status", [
    (0, binding.ATTN_EINVAL),              # no lse buffer
    (A * 256 + 2, binding.ATTN_EALIGN),    # lse not 4-byte aligned
    (A * 192 + 64, binding.ATTN_EINVAL),   # lse overlaps o
    (A + 4096, binding.ATTN_EINVAL),       # lse overlaps q
])
def test_fwd_lse_rejects_bad_lse(lse, status):
    assert _lse_call(lse) == status


def test_decode_workspace_bytes():
    """Partial outputs (fp32 x D) and (m, l) pairs per (b, hq, split): at
    least one split, at most one per 32 keys; 0 for invalid sizes."""
    ws = binding.attn_decode_workspace_bytes
    assert ws(0, 8, 2, 100, 128) == 0 and ws(1, 8, 2, 0, 128) == 0 and ws(1, 8, 2, 10, 128, -1) == 0
    one = ws(2, 8, 2, 1000, 128, 1)
    assert one >= 2 * 8 * (128 + 2) * 4
    assert ws(2, 8, 2, 1000, 128, 4) >= 4 * 2 * 8 * (128 + 2) * 4
    # at most ceil(1000 / 32) = 32 splits, whatever is asked
    assert ws(2, 8, 2, 1000, 128, 10 ** 6) == ws(2, 8, 2, 1000, 128, 32)
    assert ws(1, 64, 8, 32768, 128) > 0


def _dec_call(**kw):
    """attn_decode with fake device addresses: only argument errors caught
    before any device call are exercised here."""
    a = dict(q=A, k=A * 64, v=A * 128, o=A * 192, lse=None, ws=A * 256, nws=1 << 30, B=1, Hq=8, Hkv=2,
             L=100, D=128, theta=1e4, scale=0.088, w=None, ns=0)
    a.update(kw)
    return binding.lib().attn_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], a["nws"], a["B"],
                                     a["Hq"], a["Hkv"], a["L"], a["D"], a["theta"], a["scale"], a["w"],
                                     a["ns"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=66, Hkv=2), binding.ATTN_EUNSUPPORTED),   # 33 query heads per KV head
    (dict(D=96), binding.ATTN_EUNSUPPORTED),
    (dict(Hq=5, Hkv=2), binding.ATTN_EINVAL),
    (dict(ns=-1), binding.ATTN_EINVAL),
    (dict(ws=0), binding.ATTN_EINVAL),
    (dict(q=0), binding.ATTN_EINVAL),
    (dict(q=A + 8), binding.ATTN_EALIGN),
    (dict(ws=A * 256 + 4), binding.ATTN_EALIGN),
    (dict(lse=A * 300 + 2), binding.ATTN_EALIGN),
    (dict(scale=0.0), binding.ATTN_EINVAL),
    (dict(theta=0.5), binding.ATTN_EINVAL),
    (dict(nws=64), binding.ATTN_EINVAL),                 # workspace too small
    (dict(o=A), binding.ATTN_EINVAL),                    # o aliases q
    (dict(ws=A * 192), binding.ATTN_EINVAL),             # workspace overlaps o
])
def test_decode_rejects(kw, status):
    assert _dec_call(**kw) == status


def test_decode_empty_is_ok_without_device():
    assert _dec_call(B=0, q=0, k=0, v=0, o=0, ws=0, nws=0) == binding.ATTN_OK
    assert _dec_call(L=0, q=0, k=0, v=0, o=0, ws=0, nws=0) == binding.ATTN_OK


def test_bwd_workspace_bytes():
    """Staged queries and keys (bf16) and Delta (fp32), 256-byte aligned
    sections, plus fp32 partial dK and dV per query head of a group when the
    dK/dV grid (one work-group per 256 keys and KV head) is under 1024
    work-groups; 0 for empty or invalid sizes."""
    ws = binding.attn_bwd_workspace_bytes
    assert ws(0, 8, 2, 100, 128) == 0 and ws(1, 8, 2, 0, 128) == 0 and ws(1, 0, 2, 10, 128) == 0
    assert ws(1, 8, 3, 100, 128) == 0
    base = lambda B, Hq, Hkv, S, D: B * S * Hq * D * 2 + B * S * Hkv * D * 2 + B * Hq * S * 4
    # split: 4 tiles x 2 KV heads x 2 = 16 work-groups, each group of 4 heads split in 4
    B, Hq, Hkv, S, D = 2, 8, 2, 1000, 128
    need = base(B, Hq, Hkv, S, D) + 2 * 4 * B * S * Hkv * D * 4
    assert need <= ws(B, Hq, Hkv, S, D) <= need + 1280
    # not split: 32 tiles x 8 KV heads x 4 = 1024 work-groups
    B, Hq, Hkv, S, D = 4, 32, 8, 8192, 128
    need = base(B, Hq, Hkv, S, D)
    assert need <= ws(B, Hq, Hkv, S, D) <= need + 768
    # no groups, never split
    B, Hq, Hkv, S, D = 1, 2, 2, 300, 64
    need = base(B, Hq, Hkv, S, D)
    assert need <= ws(B, Hq, Hkv, S, D) <= need + 768


def _bwd_call(**kw):
    """attn_bwd with fake device addresses: only argument errors caught
    before any device call are exercised here."""
    a = dict(q=A, k=A * 64, v=A * 128, o=A * 192, do=A * 256, lse=A * 320, dq=A * 384, dk=A * 448, dv=A * 512,
             ws=A * 576, nws=1 << 30, B=1, Hq=8, Hkv=2, S=100, D=128, theta=1e4, causal=1, scale=0.088, w=None)
    a.update(kw)
    return binding.lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                  a["ws"], a["nws"], a["B"], a["Hq"], a["Hkv"], a["S"], a["D"], a["theta"],
                                  a["causal"], a["scale"], a["w"], None)


_W = (ctypes.c_int32 * 64)(*range(64))


@pytest.mark.parametrize("kw,status", [
    (dict(w=_W), binding.ATTN_EUNSUPPORTED),           # no backward of the window
    (dict(D=96), binding.ATTN_EUNSUPPORTED),
    (dict(B=1_600_000_000, S=512, Hq=1, Hkv=1), binding.ATTN_EINVAL),   # over 2^31 - 1 work-groups
    (dict(Hq=5, Hkv=2), binding.ATTN_EINVAL),
    (dict(causal=2), binding.ATTN_EINVAL),
    (dict(scale=-1.0), binding.ATTN_EINVAL),
    (dict(theta=0.5), binding.ATTN_EINVAL),
    (dict(do=0), binding.ATTN_EINVAL),
    (dict(lse=0), binding.ATTN_EINVAL),
    (dict(ws=0), binding.ATTN_EINVAL),
    (dict(dk=A * 448 + 8), binding.ATTN_EALIGN),
    (dict(lse=A * 320 + 2), binding.ATTN_EALIGN),
    (dict(nws=1024), binding.ATTN_EINVAL),               # workspace too small
    (dict(dq=A), binding.ATTN_EINVAL),                   # dq aliases q
    (dict(dv=A * 448), binding.ATTN_EINVAL),             # dv aliases dk
    (dict(ws=A * 320), binding.ATTN_EINVAL),             # workspace overlaps lse
])
def test_bwd_rejects(kw, status):
    assert _bwd_call(**kw) == status


def test_bwd_empty_is_ok_without_device():
    z = dict(q=0, k=0, v=0, o=0, do=0, lse=0, dq=0, dk=0, dv=0, ws=0, nws=0)
    assert _bwd_call(B=0, **z) == binding.ATTN_OK
    assert _bwd_call(S=0, **z) == binding.ATTN_OK


# ---- persistent schedule ("Croqtile", "Step 4": host task list, cost-balanced
# bins, an order inside a bin that keeps K/V reuse) -----------------------------

def _tile_cost(qt, S):
    # the 64-key tiles a causal 256-row query tile visits, plus 2 for its Q
    # load and epilogue
    return -(-min(S, (qt + 1) * 256) // 64) + 2


@pytest.mark.parametrize("B,Hq,S,bins", [
    (4, 32, 8192, 256),     # prefill_s8192: 4096 tiles over 256 bins, 8 XCD groups
    (1, 32, 16384, 256),    # gqa_s16384's 32 query heads: 2048 tiles
    (1, 32, 32768, 256),    # window_s32768's shape
    (1, 2, 256, 256),       # tiny: fewer tiles than bins -> one tile per bin
    (2, 3, 1000, 256),      # 6 heads: one group over all bins, ragged S
    (3, 8, 4000, 100),      # bin count not a multiple of 8: one group
])
def test_persistent_schedule_properties(B, Hq, S, bins):
    off, tasks = binding.attn_persistent_schedule(B, Hq, S, bins)
    n_qt = -(-S // 256)
    n_tasks = B * Hq * n_qt
    nb = min(bins, n_tasks)
    # offsets: bins' + 1 entries rising from 0 to the task count
    assert len(off) == nb + 1 and off[0] == 0 and off[-1] == n_tasks and len(tasks) == n_tasks
    assert np.all(np.diff(off.astype(np.int64)) >= 0)
    # every (b, hq, qt) exactly once
    qt, hq, b = tasks & 4095, (tasks >> 12) & 1023, tasks >> 22
    assert qt.max() < n_qt and hq.max() < Hq and b.max() < B
    flat = (b.astype(np.int64) * Hq + hq) * n_qt + qt
    assert np.array_equal(np.sort(flat), np.arange(n_tasks))
    cost = np.array([_tile_cost(int(t), S) for t in qt])
    n_bh = B * Hq
    groups = 8 if (n_bh % 8 == 0 and nb % 8 == 0) else 1
    loads = np.array([cost[off[g]:off[g + 1]].sum() for g in range(nb)])
    for x in range(groups):
        gb = list(range(x, nb, groups))
        # XCD grouping: bin g holds only the heads of group g % 8
        if groups == 8:
            h0, h1 = x * n_bh // 8, (x + 1) * n_bh // 8
            for g in gb:
                bh = b[off[g]:off[g + 1]].astype(np.int64) * Hq + hq[off[g]:off[g + 1]]
                assert np.all((bh >= h0) & (bh < h1))
        # longest-first to the lightest bin: no bin exceeds the lightest by
        # more than the largest task of the group
        gl = loads[gb]
        assert gl.max() - gl.min() <= max(cost[off[g]:off[g + 1]].max(initial=0) for g in gb)
    # inside a bin: band by band (bands of max(1, 64 // n_qt) heads), longest
    # tile first within a band
    kb = max(1, 64 // n_qt)
    band = (b.astype(np.int64) * Hq + hq) // kb
    for g in range(nb):
        key = list(zip(band[off[g]:off[g + 1]].tolist(), (-cost[off[g]:off[g + 1]]).tolist()))
        assert key == sorted(key)


def test_persistent_schedule_balance_prefill_s8192():
    """The 4096 query tiles of B4 H32 S8192 over 256 bins: every bin within
    one tile's cost of the mean (the causal costs run 6..130)."""
    off, tasks = binding.attn_persistent_schedule(4, 32, 8192, 256)
    cost = np.array([_tile_cost(int(t) & 4095, 8192) for t in tasks])
    loads = np.array([cost[off[g]:off[g + 1]].sum() for g in range(256)])
    assert loads.sum() == cost.sum()
    assert loads.max() - loads.min() <= 130
    assert loads.max() <= loads.mean() * 1.05


def test_persistent_schedule_argument_errors():
    for args in ((0, 32, 8192, 256), (4, 0, 8192, 256), (4, 32, 0, 256), (4, 32, 8192, 0)):
        with pytest.raises(binding.AttnError):
            binding.attn_persistent_schedule(*args)
    with pytest.raises(binding.AttnError) as e:
        binding.attn_persistent_schedule(1, 2000, 256, 256)     # hq does not fit 10 bits
    assert e.value.status == binding.ATTN_EUNSUPPORTED
    out = np.zeros(4, dtype=np.uint32)
    n = binding.lib().attn_persistent_schedule(1, 2, 256, 256, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), 4)
    assert n == binding.ATTN_EINVAL   # needs 3 offsets + 2 tasks = 5


def test_fwd_persistent_rejects_window():
    """attn_fwd_persistent with fake device addresses: the window and size
    limits are argument errors caught before any device call."""
    w = (ctypes.c_int32 * 64)(*([1 << 20] * 64))
    call = binding.lib().attn_fwd_persistent
    assert call(A, A * 64, A * 128, A * 192, 1, 4, 2, 128, 128, 1e4, 1, 0.088, w, None) == binding.ATTN_EUNSUPPORTED
    assert call(A, A * 64, A * 128, A * 192, 1, 2048, 2048, 1, 128, 1e4, 1, 0.088, None, None) == \
        binding.ATTN_EUNSUPPORTED
    assert call(A, A * 64, A * 128, A * 192, 1, 4, 3, 128, 128, 1e4, 1, 0.088, None, None) == binding.ATTN_EINVAL


def test_binding_rejects_host_tensors_before_any_call():
    """A host tensor's address handed to a kernel would fault the GPU: every
    wrapper rejects host tensors before it reaches the library."""
    import torch
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        binding.attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        binding.attn_fwd_lse(q, q, q)
    with pytest.raises(TypeError):
        binding.attn_fwd_persistent(q, q, q)
    with pytest.raises(TypeError):
        binding.attn_rope_apply(q, q)
    with pytest.raises(TypeError):
        binding.attn_decode(q[:, 0].contiguous(), q, q)
    with pytest.raises(TypeError):
        binding.attn_bwd(q, q, q, q, torch.zeros(1, 2, 64), q)


def _dec_noalloc_call(**kw):
    a = dict(q=A, k=A * 64, v=A * 128, o=A * 192, lse=None, B=1, Hq=8, Hkv=2, L=100, D=128, theta=1e4,
             scale=0.088, w=None, ns=0)
    a.update(kw)
    return binding.lib().attn_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                             a["L"], a["D"], a["theta"], a["scale"], a["w"], a["ns"], None)


def test_decode_noalloc_limits_and_errors():
    """The no-allocation decode takes the split partials from a static
    buffer of attn_decode_scratch_bytes(); a call that needs more is
    rejected on the host (ATTN_ESCRATCH) before any device work, and the
    argument errors are attn_decode's."""
    cap = binding.attn_decode_scratch_bytes()
    assert cap == 32 << 20
    # the library's own split plan fits the scratch for the supported groupings
    for B, Hq, Hkv, L, D in ((1, 64, 8, 32768, 128), (8, 64, 8, 32768, 128), (1, 32, 1, 1 << 20, 128),
                             (64, 64, 2, 4096, 128), (3, 12, 12, 77, 64)):
        assert binding.attn_decode_workspace_bytes(B, Hq, Hkv, L, D, 0) <= cap
    big = dict(B=64, Hq=64, Hkv=8, L=32768, D=128, ns=1024)
    assert binding.attn_decode_workspace_bytes(64, 64, 8, 32768, 128, 1024) > cap
    assert _dec_noalloc_call(**big) == binding.ATTN_ESCRATCH
    assert _dec_noalloc_call(Hq=66, Hkv=2) == binding.ATTN_EUNSUPPORTED
    assert _dec_noalloc_call(q=A + 8) == binding.ATTN_EALIGN
    assert _dec_noalloc_call(o=A) == binding.ATTN_EINVAL
    assert _dec_noalloc_call(scale=-1.0) == binding.ATTN_EINVAL
    assert _dec_noalloc_call(B=0) == binding.ATTN_OK


def test_rope_apply_keys_only_argument_rules():
    lib = binding.lib()
    # q and q_out must both be NULL or both set
    assert lib.attn_rope_apply(None, A, A * 64, A * 128, 1, 2, 2, 64, 128, 1e4, None) == binding.ATTN_EINVAL
    assert lib.attn_rope_apply(A, A * 64, None, A * 128, 1, 2, 2, 64, 128, 1e4, None) == binding.ATTN_EINVAL
    # keys only: the output must not overlap the input keys
    assert lib.attn_rope_apply(None, A, None, A, 1, 2, 2, 64, 128, 1e4, None) == binding.ATTN_EINVAL
    assert lib.attn_rope_apply(None, A, None, A * 64, 1, 2, 2, 64, 128, 0.0, None) == binding.ATTN_EINVAL


def test_fwd_rotated_k_needs_theta():
    """The query is rotated in the kernel: theta 0 is rejected before any
    device call."""
    st = binding.lib().attn_fwd_rotated_k(A, A * 64, A * 128, A * 192, 1, 2, 2, 64, 128, 0.0, 1, 0.088, None, None)
    assert st == binding.ATTN_EINVAL
