"""Build the HIP library libattn_mi355x.so in-tree for gfx950, and its
debug twin libattn_mi355x_serial.so (no direct loads in flight).

    python -m attention_attn_fwd_04_amd.build

hipcc cross-compiles without a GPU.  Every HIP source is compiled with the
packed-fp32 instructions disabled (the compiler would otherwise form
v_pk_*_f32 from ordinary float code).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Debug build: every direct-to-LDS load waited for as it is issued (no
# prefetch in flight); its outputs must be bitwise the pipelined library's.
SERIAL_LIB_PATH = os.path.join(PKG, "libattn_mi355x_serial.so")
SOURCES = ["attn_api.cpp", "attn_fwd_kernel.hip", "rope_pass.hip", "attn_decode.hip", "attn_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, serial: bool = False) -> str:
    """Build the library (serial=True: the debug build with serial loads)."""
    out = SERIAL_LIB_PATH if serial else LIB_PATH
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + (["-DATTN_SERIAL_LOADS=1"] if serial else []) + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the GPU-only feature flag.
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, serial=True))
