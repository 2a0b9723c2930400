"""Thin ctypes binding over libattn_mi355x.so (the C ABI in include/attn.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing or no gfx950
device is current, the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_mi355x.so")
# The debug twin built with every direct-to-LDS load waited for as it is
# issued; its outputs must be bitwise the pipelined library's.
SERIAL_LIB_PATH = os.path.join(_PKG, "libattn_mi355x_serial.so")

ATTN_OK = 0
ATTN_EINVAL = -1
ATTN_EUNSUPPORTED = -2
ATTN_EALIGN = -3
ATTN_ENOMEM = -4
ATTN_ELAUNCH = -5
ATTN_ENODEVICE = -6
ATTN_ESCRATCH = -7

EXPORTED = ("attn_fwd", "attn_fwd_lse", "attn_fwd_persistent", "attn_fwd_rotated_k", "attn_persistent_schedule",
            "attn_decode",
            "attn_decode_workspace_bytes", "attn_decode_noalloc", "attn_decode_scratch_bytes", "attn_bwd",
            "attn_bwd_workspace_bytes", "attn_rope_apply", "attn_window_table", "attn_pruned_terms",
            "attn_check_args", "attn_strerror", "attn_release")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, strerror(status), status))


_loaded = {}


def lib():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


class use_library:
    """Route the wrappers' calls to another build of the library (for
    example SERIAL_LIB_PATH) inside a `with` block.  It swaps the module's
    library handle, so it is for tests and single-threaded tools: calls made
    from other threads meanwhile go to the same build."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = _load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _load(path):
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError("HIP library %s is not built; run `python -m "
                           "attention_attn_fwd_04_amd.build`" % path)
    L = ctypes.CDLL(path)
    vp, i, f, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, f, i32p, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, f, i32p, vp]
    L.attn_fwd_lse.restype = i
    L.attn_fwd_persistent.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, f, i32p, vp]
    L.attn_fwd_persistent.restype = i
    L.attn_fwd_rotated_k.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, f, i32p, vp]
    L.attn_fwd_rotated_k.restype = i
    L.attn_persistent_schedule.argtypes = [i, i, i, i, ctypes.POINTER(ctypes.c_uint32), ctypes.c_longlong]
    L.attn_persistent_schedule.restype = ctypes.c_longlong
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, f, f, i32p, i, vp]
    L.attn_decode.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, i32p, i, vp]
    L.attn_decode_noalloc.restype = i
    L.attn_decode_scratch_bytes.argtypes = []
    L.attn_decode_scratch_bytes.restype = ctypes.c_size_t
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i, i, i, i, i, f, i, f, i32p, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.attn_rope_apply.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, vp]
    L.attn_rope_apply.restype = i
    L.attn_window_table.argtypes = [d, i, d, i32p]
    L.attn_window_table.restype = i
    L.attn_pruned_terms.argtypes = [i32p, i, i, ctypes.POINTER(ctypes.c_longlong)]
    L.attn_pruned_terms.restype = i
    L.attn_check_args.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, f, i32p]
    L.attn_check_args.restype = i
    L.attn_strerror.argtypes = [i]
    L.attn_strerror.restype = ctypes.c_char_p
    L.attn_release.argtypes = []
    L.attn_release.restype = None
    _loaded[path] = L
    return L


def strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def _window_ptr(window_table, D):
    if window_table is None:
        return None, None
    w = np.ascontiguousarray(np.asarray(window_table, dtype=np.int32))
    if w.shape != (D // 2,):
        raise ValueError("window_table must hold D/2 = %d int32 values" % (D // 2))
    return w, w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(t, name, like=None):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 4:
        raise TypeError("%s must be a 4-d bfloat16 tensor [B, S, H, D]" % name)
    _check_device(t, name, like)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (BSHD)" % name)


def _check_device(t, name, like=None):
    """Every tensor whose address reaches the library must live on the GPU,
    on the device of the call's first input (a host address handed to a
    kernel faults the GPU)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if like is not None and t.device != like.device:
        raise ValueError("%s must be on %s like the inputs (got %s)" % (name, like.device, t.device))


def _check_buffer(t, name, like, dtype, shape=None):
    """A device buffer the library reads or writes: dtype, device, shape and
    contiguity checked before anything is enqueued."""
    _check_device(t, name, like)
    if t.dtype != dtype:
        raise TypeError("%s must be %s" % (name, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def attn_fwd(q, k, v, o=None, *, rope_theta=10000.0, causal=True, scale=None,
             window_table=None, stream=None):
    """Fused causal attention forward with RoPE at load; returns o [B,S,Hq,D]."""
    return _fwd("attn_fwd", q, k, v, o, rope_theta, causal, scale, window_table, stream)


def attn_fwd_persistent(q, k, v, o=None, *, rope_theta=10000.0, causal=True, scale=None,
                        window_table=None, stream=None):
    """attn_fwd on the persistent, cost-balanced schedule of the causal query
    tiles; returns o [B,S,Hq,D] (bitwise equal to attn_fwd's)."""
    return _fwd("attn_fwd_persistent", q, k, v, o, rope_theta, causal, scale, window_table, stream)


def attn_fwd_rotated_k(q, k_rot, v, o=None, *, rope_theta=10000.0, causal=True, scale=None,
                       window_table=None, stream=None):
    """attn_fwd with the query rotated at load and keys already rotated
    (attn_rope_apply(None, k)); returns o [B,S,Hq,D], bitwise attn_fwd's."""
    return _fwd("attn_fwd_rotated_k", q, k_rot, v, o, rope_theta, causal, scale, window_table, stream)


def attn_persistent_schedule(B, Hq, S, bins):
    """The task list of attn_fwd_persistent for (B, Hq, S) over `bins` bins:
    (offsets [bins'+1], tasks [n]) as numpy uint32 arrays, task =
    qt | hq << 12 | b << 22."""
    import numpy as np
    n_tasks = B * Hq * ((S + 255) // 256)
    cap = min(bins, n_tasks) + 1 + n_tasks
    out = np.zeros(cap, dtype=np.uint32)
    n = lib().attn_persistent_schedule(int(B), int(Hq), int(S), int(bins),
                                       out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), cap)
    if n < 0:
        raise AttnError(int(n), "attn_persistent_schedule")
    nb = int(n) - 1 - n_tasks
    return out[:nb + 1].copy(), out[nb + 1:int(n)].copy()


def _fwd(entry, q, k, v, o, rope_theta, causal, scale, window_table, stream):
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_tensor(o, "o", q)
        if o.shape != q.shape:
            raise ValueError("o must have q's shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    w, wp = _window_ptr(window_table, D)
    st = getattr(lib(), entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, Hq, Hkv, S, D,
                               float(rope_theta), int(bool(causal)), float(scale), wp, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, entry)
    return o


def attn_fwd_lse(q, k, v, o=None, lse=None, *, rope_theta=10000.0, causal=True, scale=None,
                 window_table=None, stream=None):
    """attn_fwd plus the natural-log LSE of every row's scores; returns
    (o [B,S,Hq,D] bf16, lse [B,Hq,S] fp32)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_tensor(o, "o", q)
        if o.shape != q.shape:
            raise ValueError("o must have q's shape")
    if lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    else:
        _check_buffer(lse, "lse", q, torch.float32, (B, Hq, S))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    w, wp = _window_ptr(window_table, D)
    st = lib().attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, Hq, Hkv, S, D, float(rope_theta), int(bool(causal)), float(scale), wp,
                            _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_lse")
    return o, lse


def attn_decode_workspace_bytes(B, Hq, Hkv, L, D, num_splits=0) -> int:
    return int(lib().attn_decode_workspace_bytes(int(B), int(Hq), int(Hkv), int(L), int(D), int(num_splits)))


def attn_decode(q, k, v, o=None, lse=None, workspace=None, *, rope_theta=10000.0, scale=None,
                window_table=None, num_splits=0, want_lse=False, stream=None):
    """Split-KV decode: q [B, Hq, D] (the token at position L-1) against the
    cache k, v [B, L, Hkv, D]; returns o [B, Hq, D] (and lse [B, Hq] fp32 when
    want_lse or an lse buffer is given)."""
    import torch
    for t, n in ((k, "k"), (v, "v")):
        _check_tensor(t, n, k)
    B, L, Hkv, D = k.shape
    if v.shape != k.shape:
        raise ValueError("v must match k [B, L, Hkv, D]")
    if (not isinstance(q, torch.Tensor) or q.dtype != torch.bfloat16 or q.dim() != 3
            or q.shape[0] != B or q.shape[2] != D):
        raise ValueError("q must be a bfloat16 tensor [B, Hq, D]")
    _check_buffer(q, "q", k, torch.bfloat16)
    Hq = q.shape[1]
    if o is None:
        o = torch.empty_like(q)
    else:
        _check_buffer(o, "o", k, torch.bfloat16, q.shape)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer(lse, "lse", k, torch.float32, (B, Hq))
    nbytes = attn_decode_workspace_bytes(B, Hq, Hkv, L, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_device(workspace, "workspace", k)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    w, wp = _window_ptr(window_table, D)
    st = lib().attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                           lse.data_ptr() if lse is not None else None,
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           B, Hq, Hkv, L, D, float(rope_theta), float(scale), wp, int(num_splits),
                           _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode")
    return (o, lse) if lse is not None else o


def attn_decode_scratch_bytes() -> int:
    return int(lib().attn_decode_scratch_bytes())


def attn_decode_noalloc(q, k, v, o, lse=None, *, rope_theta=10000.0, scale=None, window_table=None,
                        num_splits=0, stream=None):
    """attn_decode without a workspace and without any allocation, by this
    wrapper or the library: the split partials live in the library's static
    device scratch.  The caller passes the output o [B, Hq, D] (and lse
    [B, Hq] fp32 if wanted); both are filled and o (or (o, lse)) returned.
    Calls that overlap on one device race on the shared scratch."""
    import torch
    for t, n in ((k, "k"), (v, "v")):
        _check_tensor(t, n, k)
    B, L, Hkv, D = k.shape
    if v.shape != k.shape:
        raise ValueError("v must match k [B, L, Hkv, D]")
    if (not isinstance(q, torch.Tensor) or q.dtype != torch.bfloat16 or q.dim() != 3
            or q.shape[0] != B or q.shape[2] != D):
        raise ValueError("q must be a bfloat16 tensor [B, Hq, D]")
    _check_buffer(q, "q", k, torch.bfloat16)
    Hq = q.shape[1]
    _check_buffer(o, "o", k, torch.bfloat16, q.shape)
    if lse is not None:
        _check_buffer(lse, "lse", k, torch.float32, (B, Hq))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    w, wp = _window_ptr(window_table, D)
    st = lib().attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, B, Hq, Hkv, L, D,
                                   float(rope_theta), float(scale), wp, int(num_splits), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_decode_noalloc")
    return (o, lse) if lse is not None else o


def attn_bwd_workspace_bytes(B, Hq, Hkv, S, D) -> int:
    return int(lib().attn_bwd_workspace_bytes(int(B), int(Hq), int(Hkv), int(S), int(D)))


def attn_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, workspace=None, *, rope_theta=10000.0,
             causal=True, scale=None, window_table=None, stream=None):
    """Attention backward: (dq, dk, dv) for the forward output o and its lse
    (attn_fwd_lse with the same arguments) and the output gradient dout."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check_tensor(t, n, q)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape:
        raise ValueError("k and v must be [B, S, Hkv, D] matching q")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    _check_buffer(lse, "lse", q, torch.float32, (B, Hq, S))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _check_tensor(t, n, q)
        if t.shape != ref.shape:
            raise ValueError("%s must be shaped like %s" % (n, "q" if ref is q else "k"))
    nbytes = attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    else:
        _check_device(workspace, "workspace", q)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    w, wp = _window_ptr(window_table, D)
    st = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                        workspace.numel() * workspace.element_size(), B, Hq, Hkv, S, D, float(rope_theta),
                        1 if causal else 0, float(scale), wp, _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_rope_apply(q, k, q_out=None, k_out=None, *, rope_theta=10000.0, stream=None):
    """Separate RoPE pass: rotated copies (q_out, k_out) of q and k.  With
    q None only the keys are rotated (q_out is then None)."""
    import torch
    _check_tensor(k, "k", k)
    B, S, Hkv, D = k.shape
    if q is not None:
        _check_tensor(q, "q", k)
        Hq = q.shape[2]
        if q.shape != (B, S, Hq, D):
            raise ValueError("k must be [B, S, Hkv, D] matching q")
        q_out = torch.empty_like(q) if q_out is None else q_out
        _check_tensor(q_out, "q_out", k)
        if q_out.shape != q.shape:
            raise ValueError("q_out must be shaped like q")
    else:
        if q_out is not None:
            raise ValueError("q_out without q")
        Hq = Hkv
    k_out = torch.empty_like(k) if k_out is None else k_out
    _check_tensor(k_out, "k_out", k)
    if k_out.shape != k.shape:
        raise ValueError("k_out must be shaped like k")
    st = lib().attn_rope_apply(q.data_ptr() if q is not None else None, k.data_ptr(),
                               q_out.data_ptr() if q is not None else None, k_out.data_ptr(),
                               B, Hq, Hkv, S, D, float(rope_theta), _stream_handle(stream))
    if st != ATTN_OK:
        raise AttnError(st, "attn_rope_apply")
    return q_out, k_out


def attn_window_table(rope_theta, D, k_turns=2.0):
    out = np.zeros(D // 2, dtype=np.int32)
    st = lib().attn_window_table(float(rope_theta), int(D), float(k_turns),
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if st != ATTN_OK:
        raise AttnError(st, "attn_window_table")
    return out


def attn_pruned_terms(window_table, D, S) -> int:
    w, wp = _window_ptr(window_table, D)
    res = ctypes.c_longlong(0)
    st = lib().attn_pruned_terms(wp, int(D), int(S), ctypes.byref(res))
    if st != ATTN_OK:
        raise AttnError(st, "attn_pruned_terms")
    return int(res.value)


def attn_check_args(q_ptr, k_ptr, v_ptr, o_ptr, B, Hq, Hkv, S, D, rope_theta, causal, scale,
                    window_table=None) -> int:
    """Raw host-side validation on integer addresses; returns the status."""
    w, wp = _window_ptr(window_table, D) if window_table is not None else (None, None)
    return int(lib().attn_check_args(q_ptr, k_ptr, v_ptr, o_ptr, B, Hq, Hkv, S, D,
                                     float(rope_theta), int(causal), float(scale), wp))


def attn_release():
    lib().attn_release()
