"""Wait-state check of the built library's LDS-DMA loads (CPU only).

The kernels issue their direct-to-LDS buffer loads (`buffer_load_dwordx4 ...
offen lds`) through inline assembly, and the compiler does not check hazards
on the scalar operands of an inline-assembly statement.  On gfx9-family
parts (gfx950 included) two manual wait-state rules apply to these loads:

  * a VALU instruction that writes an SGPR (v_readfirstlane, v_readlane,
    v_cmp into an SGPR pair) needs 5 wait states before a VMEM instruction
    reads that SGPR: here the buffer descriptor;
  * an SALU write of M0 needs 1 wait state before an LDS DMA, which takes its
    LDS address from M0.

A load that reads a descriptor word too early takes the register's previous
value, which may be another buffer's base address: the load then reads out
of bounds.  This test disassembles the code object of the built library
(our own build, with the ROCm LLVM tools) and checks every LDS-DMA load
against both rules.
"""
import os
import re
import subprocess
import tempfile

import pytest

from attention_attn_fwd_04_amd import binding

LLVM = "/opt/rocm/llvm/bin"


def _sgprs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _writes(ops):
    """Destination register name(s) of an instruction: the first operand."""
    return ops[0] if ops else ""


def code_objects(lib_path):
    """The gfx950 code objects of a built library: its .hip_fatbin section
    holds one offload bundle per HIP source file (magic, entry count, then
    offset / size / target triple per entry, offsets from the bundle's
    start)."""
    import struct
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fatbin.bin")
        subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib_path, fat], check=True)
        with open(fat, "rb") as f:
            data = f.read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out, pos = [], 0
    while True:
        i = data.find(magic, pos)
        if i < 0:
            break
        (n,) = struct.unpack_from("<Q", data, i + len(magic))
        off = i + len(magic) + 8
        for _ in range(n):
            o, size, tlen = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + tlen].decode()
            off += tlen
            if triple.endswith("gfx950") and size > 0:
                out.append(data[i + o:i + o + size])
        pos = i + len(magic)
    return out


def _disassembly():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    if not os.path.exists(os.path.join(LLVM, "llvm-objdump")):
        pytest.skip("ROCm LLVM tools not found")
    texts = []
    with tempfile.TemporaryDirectory() as d:
        for j, co in enumerate(code_objects(binding.LIB_PATH)):
            path = os.path.join(d, "code%d.co" % j)
            with open(path, "wb") as f:
                f.write(co)
            texts.append(subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", path],
                                        check=True, capture_output=True, text=True).stdout)
    return "\n".join(texts)


def _scan(text):
    """Yield (kernel, load, offending instruction, wait states) for every
    LDS-DMA load that breaks one of the two rules."""
    insts = []          # (kernel, mnemonic, operands, text)
    kernel = None
    for line in text.split("\n"):
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            kernel = m.group(1)
            continue
        body = line.split("//")[0].strip()
        if not body or body.endswith(":"):
            continue
        parts = body.replace(",", " ").split()
        insts.append((kernel, parts[0], parts[1:], body))
    for i, (kern, op, ops, body) in enumerate(insts):
        if not (op.startswith("buffer_load") and "lds" in ops):
            continue
        regs = set()
        for t in ops:
            regs |= _sgprs(t)
        ws, j = 0, i - 1
        while j >= 0 and ws < 5 and insts[j][0] == kern:
            _, pop, pops, pbody = insts[j]
            j -= 1
            if pop == "s_nop":
                ws += int(pops[0], 0) + 1 if pops else 1
                continue
            dst = _writes(pops)
            if pop.startswith("v_") and _sgprs(dst) & regs:
                yield kern, body, pbody, ws
            if pop.startswith("s_") and dst == "m0" and ws < 1:
                yield kern, body, pbody, ws
            if pop.startswith(("s_cbranch", "s_branch", "s_setpc", "s_swappc")):
                break
            ws += 1


def test_scanner_flags_a_planted_hazard():
    text = ("0000000000001000 <k>:\n"
            "\tv_readfirstlane_b32 s41, v3\n"
            "\ts_nop 0\n"
            "\tbuffer_load_dwordx4 v6, s[40:43], 0 offen lds\n"
            "\ts_mov_b32 m0, s2\n"
            "\tbuffer_load_dwordx4 v6, s[44:47], 0 offen lds\n"
            "\tv_readfirstlane_b32 s41, v3\n"
            "\ts_nop 4\n"
            "\tbuffer_load_dwordx4 v6, s[40:43], 0 offen lds\n")
    found = list(_scan(text))
    assert len(found) == 2
    assert found[0][3] == 1 and "s41" in found[0][2]
    assert "m0" in found[1][2]


def test_every_source_file_is_scanned():
    """One code object per HIP source file, and the direct-to-LDS loads of
    the forward, decode and backward kernels are all in the scan."""
    text = _disassembly()
    assert len(code_objects(binding.LIB_PATH)) == 4
    for kernel in ("attn_fwd_kernel", "decode_split_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"):
        assert kernel in text, kernel
    loads = [l for l in text.split("\n") if "buffer_load" in l and " lds" in l]
    assert len(loads) > 700, len(loads)


def test_lds_dma_wait_states():
    found = list(_scan(_disassembly()))
    for f in found[:10]:
        print(f)
    assert not found, "%d LDS-DMA loads break a wait-state rule" % len(found)
