"""ctypes front end of the fp64 CPU oracle (attn_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only callers.  The product path never imports this
module, and this module imports nothing from the product package.

Tensors are numpy uint16 arrays holding bf16 bit patterns in [B, S, H, D]
layout (the same bits the GPU path receives).  Results are fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_attn.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile attn_oracle.c with gcc into oracle/liboracle_attn.so."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_attn_rows.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                     i32p, ctypes.c_longlong, i32p, ctypes.c_longlong,
                                     f64p, f64p]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                  i32p, ctypes.c_longlong, f64p, f64p]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_attn_bwd.argtypes = [u16p, u16p, u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                    f64p, f64p, f64p]
    lib.oracle_attn_bwd.restype = ctypes.c_int
    lib.oracle_attn_bwd_sampled.argtypes = [u16p, u16p, u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                            ctypes.c_double, i32p, ctypes.c_int, f64p, i32p, ctypes.c_int, f64p,
                                            f64p]
    lib.oracle_attn_bwd_sampled.restype = ctypes.c_int
    lib.oracle_scores_row.argtypes = [u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                      ctypes.c_int, ctypes.c_double, i32p,
                                      ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, f64p]
    lib.oracle_scores_row.restype = ctypes.c_int
    lib.oracle_rope_row.argtypes = [u16p, ctypes.c_int, ctypes.c_double, ctypes.c_double, f64p]
    lib.oracle_rope_row.restype = None
    lib.oracle_window_table.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double, i32p]
    lib.oracle_window_table.restype = ctypes.c_int
    lib.oracle_pruned_terms.argtypes = [i32p, ctypes.c_int, ctypes.c_int]
    lib.oracle_pruned_terms.restype = ctypes.c_longlong
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a: np.ndarray):
    assert a.dtype == np.uint16 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def _window_arg(window, D):
    if window is None:
        return None, None
    w = np.ascontiguousarray(np.asarray(window, dtype=np.int32))
    assert w.shape == (D // 2,)
    return w, w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def attn_rows(q, k, v, rows, rope_theta, causal, scale, window=None, pos_offset=0,
              want_lse=False):
    """Attention output (fp64) for the query rows `rows` = [(b, n, hq), ...].

    q: uint16 [B,S,Hq,D]; k, v: uint16 [B,S,Hkv,D].  Returns [len(rows), D]
    (and the natural-log LSE per row when want_lse)."""
    lib = _load()
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    n = rows.shape[0]
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64) if want_lse else None
    w, wp = _window_arg(window, D)
    rc = lib.oracle_attn_rows(_u16(q), _u16(k), _u16(v), B, S, Hq, Hkv, D,
                              float(rope_theta), int(bool(causal)), float(scale), wp,
                              int(pos_offset), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                              n, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                              lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_lse else None)
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return (out, lse) if want_lse else out


def decode(q, k, v, rope_theta, scale, window=None, pos_offset=0, want_lse=False):
    """Decode attention (fp64): q uint16 [B, Hq, D] at position L-1 against the
    cache k, v uint16 [B, L, Hkv, D] (keys used as stored).  Returns
    [B, Hq, D] (and the natural-log LSE [B, Hq] when want_lse)."""
    lib = _load()
    B, Hq, D = q.shape
    L, Hkv = k.shape[1], k.shape[2]
    assert k.shape == (B, L, Hkv, D) and v.shape == k.shape
    q, k, v = (np.ascontiguousarray(t) for t in (q, k, v))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64) if want_lse else None
    w, wp = _window_arg(window, D)
    rc = lib.oracle_decode(_u16(q), _u16(k), _u16(v), B, L, Hq, Hkv, D, float(rope_theta), float(scale),
                           wp, int(pos_offset), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                           lse.ctypes.data_as(ctypes.POINTER(ctypes.c_double)) if want_lse else None)
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return (out, lse) if want_lse else out


def attn_bwd(q, k, v, do, rope_theta, causal, scale):
    """Gradients (fp64) of the attention with respect to q, k, v for the
    upstream gradient do (uint16 bf16 bits, [B,S,Hq,D]).  Returns dq, dk, dv."""
    lib = _load()
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape and do.shape == q.shape
    q, k, v, do = (np.ascontiguousarray(t) for t in (q, k, v, do))
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(k.shape, dtype=np.float64)
    f = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = lib.oracle_attn_bwd(_u16(q), _u16(k), _u16(v), _u16(do), B, S, Hq, Hkv, D, float(rope_theta),
                             int(bool(causal)), float(scale), f(dq), f(dk), f(dv))
    if rc != 0:
        raise ValueError("oracle_attn_bwd rejected its arguments")
    return dq, dk, dv


def attn_bwd_sampled(q, k, v, do, rope_theta, causal, scale, qrows, kcols):
    """Single entries of attn_bwd at any size: dq of the query rows qrows
    ((b, n, hq) triples) and dk, dv of the key rows kcols ((b, m, hk)).
    Returns dq [len(qrows), D], dk, dv [len(kcols), D] (fp64)."""
    lib = _load()
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    assert k.shape == (B, S, Hkv, D) and v.shape == k.shape and do.shape == q.shape
    q, k, v, do = (np.ascontiguousarray(t) for t in (q, k, v, do))
    qr = np.ascontiguousarray(np.asarray(qrows, dtype=np.int32).reshape(-1, 3))
    kc = np.ascontiguousarray(np.asarray(kcols, dtype=np.int32).reshape(-1, 3))
    dq = np.zeros((len(qr), D), dtype=np.float64)
    dk = np.zeros((len(kc), D), dtype=np.float64)
    dv = np.zeros((len(kc), D), dtype=np.float64)
    f = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    i = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = lib.oracle_attn_bwd_sampled(_u16(q), _u16(k), _u16(v), _u16(do), B, S, Hq, Hkv, D, float(rope_theta),
                                     int(bool(causal)), float(scale), i(qr), len(qr), f(dq), i(kc), len(kc),
                                     f(dk), f(dv))
    if rc != 0:
        raise ValueError("oracle_attn_bwd_sampled rejected its arguments")
    return dq, dk, dv


def all_rows(B, S, Hq):
    b, n, h = np.meshgrid(np.arange(B), np.arange(S), np.arange(Hq), indexing="ij")
    return np.stack([b.ravel(), n.ravel(), h.ravel()], axis=1).astype(np.int32)


def attn_full(q, k, v, rope_theta, causal, scale, window=None, pos_offset=0):
    """Whole output tensor [B,S,Hq,D] in fp64."""
    B, S, Hq, D = q.shape
    out = attn_rows(q, k, v, all_rows(B, S, Hq), rope_theta, causal, scale, window,
                    pos_offset)
    return out.reshape(B, S, Hq, D)


def scores_row(q, k, b, n, hq, rope_theta, causal, scale, window=None, pos_offset=0):
    lib = _load()
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    out = np.zeros(S, dtype=np.float64)
    w, wp = _window_arg(window, D)
    rc = lib.oracle_scores_row(_u16(q), _u16(k), B, S, Hq, Hkv, D, float(rope_theta),
                               int(bool(causal)), float(scale), wp, int(pos_offset),
                               int(b), int(n), int(hq),
                               out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    if rc != 0:
        raise ValueError("oracle_scores_row rejected its arguments")
    return out


def rope_row(x_u16, rope_theta, pos):
    lib = _load()
    x = np.ascontiguousarray(x_u16, dtype=np.uint16)
    D = x.shape[0]
    out = np.zeros(D, dtype=np.float64)
    lib.oracle_rope_row(_u16(x), D, float(rope_theta), float(pos),
                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def window_table(rope_theta, D, k_turns):
    lib = _load()
    w = np.zeros(D // 2, dtype=np.int32)
    rc = lib.oracle_window_table(float(rope_theta), int(D), float(k_turns),
                                 w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != 0:
        raise ValueError("oracle_window_table rejected its arguments")
    return w


def pruned_terms(window, D, S) -> int:
    lib = _load()
    w = np.ascontiguousarray(np.asarray(window, dtype=np.int32))
    return int(lib.oracle_pruned_terms(w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                       int(D), int(S)))


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
