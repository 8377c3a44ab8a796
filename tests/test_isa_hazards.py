"""Machine-code check of the built library (CPU only): no MFMA accumulates
directly onto the fresh result of an MFMA of another shape.

On MI355X a v_mfma_f32_16x16x16_bf16 that takes as its accumulator input
(source C) the result of a v_mfma_f32_16x16x32_bf16 issued just before it
returned wrong values: the compiler separates the two shapes by no wait
states.  (Found as wrong outputs, with the states right, in builds whose
output tiles summed the 16x16x16 term P U onto the 16x16x32 terms Q S; two
accumulators and a VALU add fixed them.)  The kernels therefore never chain
two shapes through one accumulator without another MFMA in between.  This
test disassembles every gfx950 code object in libkda.so (code built here)
and checks that rule on the instruction stream.
"""
import os
import re
import shutil
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_recurrent_attention_chunkwise_amd", "libkda.so")
LLVM = "/opt/rocm/llvm/bin"
MFMA = re.compile(r"^\s*(v_mfma_\S+)\s+([va]\[\d+:\d+\]),\s*([^,]+),\s*([^,]+),\s*(\S+)")
BRANCH = re.compile(r"^\s*s_(cbranch_\w+|branch|setpc_b64|endpgm)\b")
FUNC = re.compile(r"^[0-9a-f]+ <(\S+)>:")


def _code_objects(tmp):
    out = os.path.join(tmp, "fatbin")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={out}",
                    LIB, os.path.join(tmp, "lib.copy")], check=True)
    data = open(out, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    objs, pos = [], 0
    while (i := data.find(magic, pos)) >= 0:
        off = i + len(magic)
        (num,) = struct.unpack_from("<Q", data, off)
        off += 8
        for _ in range(num):
            eoff, esize, tlen = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + tlen].decode()
            off += tlen
            if "gfx950" in triple and esize > 0:
                path = os.path.join(tmp, f"co{len(objs)}.o")
                open(path, "wb").write(data[i + eoff:i + eoff + esize])
                objs.append(path)
        pos = i + 1
    return objs


def mixed_shape_chains(asm_text):
    """(function, producer, consumer) for every MFMA whose source C is the
    destination of the previous MFMA when that one has another opcode."""
    bad, func, prev = [], None, None
    for line in asm_text.splitlines():
        m = FUNC.match(line)
        if m:
            func, prev = m.group(1), None
            continue
        if BRANCH.match(line):
            prev = None
            continue
        m = MFMA.match(line)
        if not m:
            continue
        op, dst, _, _, srcc = m.groups()
        if prev and prev[0] != op and srcc == prev[1]:
            bad.append((func, prev[0], op))
        prev = (op, dst)
    return bad


def test_scanner_flags_the_pattern():
    asm = """0000 <k>:
\tv_mfma_f32_16x16x32_bf16 v[34:37], v[62:65], v[70:73], v[34:37]
\ts_waitcnt lgkmcnt(1)
\tv_mfma_f32_16x16x16_bf16 v[34:37], v[0:1], v[110:111], v[34:37]
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], 0
\tv_mfma_f32_16x16x32_bf16 a[4:7], v[0:3], v[4:7], 0
\tv_mfma_f32_16x16x16_bf16 a[0:3], v[0:1], v[2:3], a[0:3]
"""
    assert mixed_shape_chains(asm) == [("k", "v_mfma_f32_16x16x32_bf16",
                                        "v_mfma_f32_16x16x16_bf16")]


def test_library_has_no_mixed_shape_chains(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in ("llvm-objcopy", "llvm-objdump")):
        pytest.skip("ROCm LLVM tools not found")
    objs = _code_objects(str(tmp_path))
    assert objs, "no gfx950 code object in libkda.so"
    bad, nmfma = [], 0
    for co in objs:
        asm = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                             check=True, capture_output=True, text=True).stdout
        nmfma += asm.count("v_mfma")
        bad += mixed_shape_chains(asm)
    assert nmfma > 1000
    assert not bad, bad[:10]
