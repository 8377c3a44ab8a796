"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, and rejects bad arguments with the documented status
before anything could be launched.  Pointers here are fake, aligned addresses
that are never dereferenced (validation runs before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "linear_recurrent_attention_chunkwise_amd", "libkda.so")

OK, NULL, SHAPE, UNSUP, MISALIGNED, ALIAS, WORKSPACE = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    from linear_recurrent_attention_chunkwise_amd import kda as binding
    return binding._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted([
        "kda_abi_version", "kda_status_str", "kda_prefill_workspace_size",
        "kda_prefill", "kda_prefill_ex", "kda_prefill_varlen",
        "kda_prefill_varlen_workspace_size", "kda_decode_step"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 3
    for s in range(8):
        assert lib.kda_status_str(s).decode().startswith("KDA_")
    assert lib.kda_status_str(99) == b"unknown kda_status"
    assert lib.kda_prefill_workspace_size(BF16, 1, 4096, 96, 128, 128, 16) == 0


BASE = 0x10_0000_0000  # fake, 16-byte aligned device addresses


def P(i, off=0):
    return ctypes.c_void_p(BASE + i * 0x1_0000_0000 + off)


def prefill(lib, dtype=BF16, B=1, T=64, H=2, dk=128, dv=128, chunk=16, ptrs=None,
            dvb=0):
    p = {n: P(i) for i, n in enumerate(["q", "k", "v", "z", "beta", "A", "S0", "o", "S_T"])}
    if ptrs:
        p.update(ptrs)
    return lib.kda_prefill_ex(dtype, B, T, H, dk, dv, chunk, p["q"], p["k"], p["v"], p["z"],
                              p["beta"], p["A"], p["S0"], p["o"], p["S_T"], None, 0, None, dvb)


def decode(lib, dtype=BF16, B=2, H=2, dk=128, dv=128, ptrs=None):
    p = {n: P(i) for i, n in enumerate(["q", "k", "v", "z", "beta", "A", "S", "o"])}
    if ptrs:
        p.update(ptrs)
    return lib.kda_decode_step(dtype, B, H, dk, dv, p["q"], p["k"], p["v"], p["z"], p["beta"],
                               p["A"], p["S"], p["o"], None)


def test_prefill_shape_and_support_errors(lib):
    assert prefill(lib, B=-1) == SHAPE
    assert prefill(lib, T=-5) == SHAPE
    assert prefill(lib, dk=0) == SHAPE
    assert prefill(lib, dtype=7) == UNSUP
    assert prefill(lib, dk=64, dv=64) == UNSUP
    assert prefill(lib, dk=128, dv=16) == UNSUP
    assert prefill(lib, chunk=32) == UNSUP
    assert prefill(lib, dvb=48) == UNSUP
    assert prefill(lib, dtype=F32, chunk=64) == UNSUP      # fp32 with dk=128 runs chunk 16
    assert prefill(lib, chunk=64, dvb=16) == UNSUP         # one-wave 64-token variant not built
    assert prefill(lib, B=1 << 40, T=1 << 40) == SHAPE     # element count overflows


def test_prefill_null_and_alignment_errors(lib):
    for name in ["q", "k", "v", "z", "beta", "o", "A", "S_T"]:
        assert prefill(lib, ptrs={name: None}) == NULL, name
    for name in ["q", "k", "v", "z", "beta", "o", "A", "S0", "S_T"]:
        assert prefill(lib, ptrs={name: P(20, 8)}) == MISALIGNED, name


def test_prefill_alias_rules(lib):
    # o overlapping an input
    assert prefill(lib, ptrs={"o": P(0, 64)}) == ALIAS
    # S_T partially overlapping S0
    assert prefill(lib, ptrs={"S_T": P(6, 16)}) == ALIAS
    # S_T overlapping o
    assert prefill(lib, ptrs={"S_T": P(7, 16)}) == ALIAS
    # S_T == S0 exactly is the allowed in-place carry; with B*H = 0 nothing launches
    assert prefill(lib, B=0, ptrs={"S_T": P(6)}) == OK


def test_prefill_empty_work_launches_nothing(lib):
    assert prefill(lib, B=0) == OK
    assert prefill(lib, H=0) == OK
    # T = 0 allows NULL token tensors (no token data exists)
    nul = {n: None for n in ["q", "k", "v", "z", "beta", "o"]}
    assert prefill(lib, B=0, T=0, ptrs=nul) == OK


def test_decode_errors(lib):
    assert decode(lib, B=-1) == SHAPE
    assert decode(lib, dk=64, dv=64) == UNSUP
    assert decode(lib, dtype=3) == UNSUP
    for name in ["q", "k", "v", "z", "beta", "A", "S", "o"]:
        assert decode(lib, ptrs={name: None}) == NULL, name
        assert decode(lib, ptrs={name: P(30, 4)}) == MISALIGNED, name
    assert decode(lib, ptrs={"o": P(6, 32)}) == ALIAS       # o inside S
    assert decode(lib, ptrs={"S": P(0, 0)}) == ALIAS        # S over q
    assert decode(lib, B=0) == OK


def varlen(lib, dtype=BF16, N=2, T=64, H=2, dk=128, dv=128, chunk=16, every=0, n_ckpt=0,
           ptrs=None, dvb=0):
    names = ["q", "k", "v", "z", "beta", "A", "S0", "o", "S_T", "cu", "ckpt", "ws"]
    p = {n: P(i) for i, n in enumerate(names)}
    if ptrs:
        p.update(ptrs)
    ws_bytes = lib.kda_prefill_varlen_workspace_size(N)
    return lib.kda_prefill_varlen(dtype, N, T, H, dk, dv, chunk, p["cu"], p["q"], p["k"],
                                  p["v"], p["z"], p["beta"], p["A"], p["S0"], p["o"],
                                  p["S_T"], every, p["ckpt"], n_ckpt, p["ws"], ws_bytes, None,
                                  dvb)


def test_varlen_argument_errors(lib):
    assert varlen(lib, N=-1) == SHAPE
    assert varlen(lib, every=-16) == SHAPE
    assert varlen(lib, every=16, n_ckpt=-1) == SHAPE
    assert varlen(lib, ptrs={"cu": None}) == NULL            # N > 0 needs offsets
    assert varlen(lib, every=16, n_ckpt=4, ptrs={"ckpt": None}) == NULL
    assert varlen(lib, every=24) == UNSUP                    # not a multiple of the chunk
    assert varlen(lib, chunk=64, every=32) == UNSUP
    assert varlen(lib, ptrs={"cu": P(20, 4)}) == MISALIGNED  # int64 offsets need 8 bytes
    assert varlen(lib, every=16, n_ckpt=4, ptrs={"ckpt": P(20, 8)}) == MISALIGNED
    # checkpoints overlapping the outputs, the initial state or an input
    assert varlen(lib, every=16, n_ckpt=4, ptrs={"ckpt": P(7, 64)}) == ALIAS
    assert varlen(lib, every=16, n_ckpt=4, ptrs={"ckpt": P(6, 64)}) == ALIAS
    assert varlen(lib, every=16, n_ckpt=4, ptrs={"ckpt": P(0, 64)}) == ALIAS
    assert varlen(lib, ptrs={"o": P(9, 0)}) == ALIAS         # o over the offsets
    # the longest-first ranking needs its workspace
    assert lib.kda_prefill_varlen_workspace_size(1) == 0
    assert lib.kda_prefill_varlen_workspace_size(2) >= 8
    assert varlen(lib, ptrs={"ws": None}) == WORKSPACE
    assert varlen(lib, ptrs={"ws": P(11, 8)}) == MISALIGNED
    assert varlen(lib, ptrs={"ws": P(7, 16)}) == ALIAS       # workspace over the outputs
    # checkpoints at 64-token chunks: not with 64 value columns per workgroup
    assert varlen(lib, chunk=64, every=64, n_ckpt=4, dvb=64) == UNSUP


def test_varlen_empty_work_launches_nothing(lib):
    assert varlen(lib, N=0, ptrs={"cu": None}) == OK
    assert varlen(lib, H=0) == OK
    # without checkpoints the checkpoint buffer is not looked at
    assert varlen(lib, N=0, every=0, n_ckpt=5, ptrs={"ckpt": P(7, 64)}) == OK
