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
# KDA_TEST_LIB: another build of the library to check (test_sanitizers.py runs
# this file against a host-sanitized build)
LIB = os.environ.get("KDA_TEST_LIB") or os.path.join(ROOT, "linear_recurrent_attention_chunkwise_amd",
                                                      "libkda.so")

OK, NULL, SHAPE, UNSUP, MISALIGNED, ALIAS, WORKSPACE = 0, 1, 2, 3, 4, 5, 6
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libkda.so is not built (run __graft_entry__.build())")
    from linear_recurrent_attention_chunkwise_amd import kda as binding
    if os.environ.get("KDA_TEST_LIB"):
        binding.library_path = lambda: LIB
    return binding._load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted([
        "kda_abi_version", "kda_status_str", "kda_prefill_workspace_size",
        "kda_prefill", "kda_prefill_ex", "kda_prefill_varlen",
        "kda_prefill_varlen_workspace_size", "kda_prefill_varlen_noalloc", "kda_decode_step",
        "kda_conv_norm",
        "kda_prefill_conv_workspace_size", "kda_prefill_conv", "kda_decode_step_conv",
        "kda_prefill_split", "kda_prefill_split_workspace_size", "kda_conv_norm_varlen",
        "kda_prefill_bwd", "kda_prefill_bwd_ex", "kda_prefill_bwd_workspace_size"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 8
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
    assert prefill(lib, B=1 << 14, T=1, H=1 << 7) == SHAPE  # 2^21 heads: grid work-items overflow
    # a 64-token tile of rows (H*d elements each) must stay below 2^31 bytes
    assert prefill(lib, B=1, T=1, H=1 << 17) == SHAPE
    assert prefill(lib, B=1, T=1, H=1 << 17, chunk=64) == SHAPE


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
    assert decode(lib, B=1 << 16, H=1 << 7) == SHAPE       # 2^23 heads x 512 work-items
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


def test_varlen_empty_work_launches_nothing(lib):
    assert varlen(lib, N=0, ptrs={"cu": None}) == OK
    assert varlen(lib, H=0) == OK
    # without checkpoints the checkpoint buffer is not looked at
    assert varlen(lib, N=0, every=0, n_ckpt=5, ptrs={"ckpt": P(7, 64)}) == OK


# ------------------------------------------------------------- prologue ----

def _addr(i):
    """Fake device address: an int is a slot index for P(), a c_void_p is used as is."""
    if i is None:
        return None
    return i.value if isinstance(i, ctypes.c_void_p) else P(i).value


def short_conv(W=4, act=0, eps=1e-6, reserved=0, w=(40, 41, 42)):
    from linear_recurrent_attention_chunkwise_amd.kda import ShortConv
    return ShortConv(W, act, eps, reserved, *[_addr(i) for i in w])


def states(*idx):
    return (ctypes.c_void_p * 3)(*[_addr(i) for i in idx])


def conv_norm(lib, dtype=BF16, B=2, T=64, H=2, dk=128, dv=128, conv=None, sin=None,
              sout=None, ptrs=None):
    p = {n: P(i) for i, n in enumerate(["q", "k", "v", "qo", "ko", "vo"])}
    if ptrs:
        p.update(ptrs)
    cs = conv if conv is not None else short_conv()
    return lib.kda_conv_norm(dtype, B, T, H, dk, dv, ctypes.byref(cs), p["q"], p["k"], p["v"],
                             sin, sout, p["qo"], p["ko"], p["vo"], None)


def test_conv_norm_argument_errors(lib):
    assert conv_norm(lib, B=-1) == SHAPE
    assert conv_norm(lib, B=1, T=1, H=1 << 17) == SHAPE   # 64-token tile past 2^31 bytes
    # 2^24 workgroups of 256 work-items (8-token tiles at bf16 d = 128): the
    # dispatch's 32-bit work-item count would wrap
    assert conv_norm(lib, B=1, T=1 << 21, H=1024) == SHAPE
    assert conv_norm(lib, dk=64, dv=64) == UNSUP
    assert conv_norm(lib, dk=128, dv=16) == UNSUP
    for bad in (short_conv(W=0), short_conv(W=5), short_conv(act=2), short_conv(eps=-1.0),
                short_conv(eps=float("nan")), short_conv(eps=float("inf")),
                short_conv(reserved=1)):
        assert conv_norm(lib, conv=bad) == UNSUP
    assert lib.kda_conv_norm(BF16, 1, 4, 2, 128, 128, None, P(0), P(1), P(2), None, None,
                             P(3), P(4), P(5), None) == NULL
    assert conv_norm(lib, conv=short_conv(w=(40, None, 42))) == NULL
    assert conv_norm(lib, ptrs={"vo": None}) == NULL
    assert conv_norm(lib, sin=states(50, None, 52)) == NULL       # all three or none
    assert conv_norm(lib, sout=states(50, 51, None)) == NULL
    assert conv_norm(lib, ptrs={"ko": P(20, 8)}) == MISALIGNED
    assert conv_norm(lib, conv=short_conv(w=(40, P(21, 4), 42))) == MISALIGNED
    assert conv_norm(lib, sin=states(50, P(51, 8), 52)) == MISALIGNED
    # outputs overlapping an input, each other, the taps or the state inputs
    assert conv_norm(lib, ptrs={"qo": P(1, 64)}) == ALIAS
    assert conv_norm(lib, ptrs={"ko": P(3, 16)}) == ALIAS
    assert conv_norm(lib, sin=states(50, 51, 52), sout=states(53, 51, 55)) == ALIAS
    assert conv_norm(lib, sout=states(53, 54, 40)) == ALIAS
    assert conv_norm(lib, sout=states(53, 54, 3)) == ALIAS
    # nothing to do
    assert conv_norm(lib, B=0) == OK
    assert conv_norm(lib, H=0, conv=short_conv(w=(None, None, None))) == OK
    # width 1 has no state: the arrays are not read
    assert conv_norm(lib, B=0, conv=short_conv(W=1), sin=states(None, None, None)) == OK
    assert conv_norm(lib, B=0, conv=short_conv(W=1), sout=states(0, 1, 2)) == OK


def test_conv_workspace_size(lib):
    n = 2 * 64 * 2 * 128 * 2
    assert lib.kda_prefill_conv_workspace_size(BF16, 2, 64, 2, 128, 128, 16) == 3 * n
    assert lib.kda_prefill_conv_workspace_size(F32, 1, 3, 1, 16, 16, 16) == 3 * 256
    assert lib.kda_prefill_conv_workspace_size(7, 1, 3, 1, 16, 16, 16) == 0
    assert lib.kda_prefill_conv_workspace_size(BF16, -1, 3, 1, 16, 16, 16) == 0


def prefill_conv(lib, dtype=BF16, B=2, T=64, H=2, dk=128, dv=128, chunk=16, conv=None,
                 sin=None, sout=None, ptrs=None, ws_bytes=None, dvb=0):
    names = ["q", "k", "v", "z", "beta", "A", "S0", "o", "S_T", "ws"]
    p = {n: P(i) for i, n in enumerate(names)}
    if ptrs:
        p.update(ptrs)
    cs = conv if conv is not None else short_conv()
    if ws_bytes is None:
        ws_bytes = lib.kda_prefill_conv_workspace_size(dtype, B, T, H, dk, dv, chunk)
    return lib.kda_prefill_conv(dtype, B, T, H, dk, dv, chunk, ctypes.byref(cs), p["q"], p["k"],
                                p["v"], p["z"], p["beta"], p["A"], sin, sout, p["S0"], p["o"],
                                p["S_T"], p["ws"], ws_bytes, None, dvb)


def test_prefill_conv_argument_errors(lib):
    assert prefill_conv(lib, T=-1) == SHAPE
    assert prefill_conv(lib, chunk=32) == UNSUP
    assert prefill_conv(lib, conv=short_conv(W=7)) == UNSUP
    assert prefill_conv(lib, ptrs={"ws": None}) == WORKSPACE
    assert prefill_conv(lib, ws_bytes=1024) == WORKSPACE
    assert prefill_conv(lib, ptrs={"ws": P(9, 8)}) == MISALIGNED
    assert prefill_conv(lib, ptrs={"z": None}) == NULL
    assert prefill_conv(lib, ptrs={"q": None}) == NULL
    # workspace over an input or an output; state out over a state in
    assert prefill_conv(lib, ptrs={"ws": P(0, 256)}) == ALIAS
    assert prefill_conv(lib, ptrs={"ws": P(7, 0)}) == ALIAS
    assert prefill_conv(lib, sin=states(50, 51, 52), sout=states(52, 53, 54)) == ALIAS
    assert prefill_conv(lib, sout=states(53, 54, 4)) == ALIAS
    # the in-place recurrent state carry stays allowed
    assert prefill_conv(lib, B=0, ptrs={"S_T": P(6)}) == OK


def decode_conv(lib, dtype=BF16, B=2, H=2, dk=128, dv=128, conv=None, st="default",
                ptrs=None):
    p = {n: P(i) for i, n in enumerate(["q", "k", "v", "z", "beta", "A", "S", "o"])}
    if ptrs:
        p.update(ptrs)
    cs = conv if conv is not None else short_conv()
    sarr = states(50, 51, 52) if st == "default" else st
    return lib.kda_decode_step_conv(dtype, B, H, dk, dv, ctypes.byref(cs), p["q"], p["k"],
                                    p["v"], p["z"], p["beta"], p["A"], sarr, p["S"], p["o"], None)


def test_decode_conv_argument_errors(lib):
    assert decode_conv(lib, B=-1) == SHAPE
    assert decode_conv(lib, dk=64, dv=64) == UNSUP
    assert decode_conv(lib, conv=short_conv(act=5)) == UNSUP
    assert decode_conv(lib, st=None) == NULL                 # W > 1 needs the states
    assert decode_conv(lib, st=states(50, None, 52)) == NULL
    assert decode_conv(lib, B=0, conv=short_conv(W=1), st=None) == OK   # no state at W = 1
    assert decode_conv(lib, st=states(50, 51, P(53, 4))) == MISALIGNED
    assert decode_conv(lib, st=states(50, 51, 6)) == ALIAS           # a state over S
    assert decode_conv(lib, st=states(50, 50, 52)) == ALIAS          # two states at once
    assert decode_conv(lib, st=states(50, 51, 40)) == ALIAS          # a state over taps
    assert decode_conv(lib, B=0) == OK


# ------------------------------------------------------- sequence split ----

def split(lib, dtype=BF16, B=1, T=4096, H=2, dk=128, dv=128, chunk=16, P=4, ptrs=None,
          ws_bytes=None):
    names = ["q", "k", "v", "z", "beta", "A", "S0", "o", "S_T", "ws"]
    p = {n: P_(i) for i, n in enumerate(names)}
    if ptrs:
        p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.kda_prefill_split_workspace_size(dtype, B, T, H, dk, dv, chunk, P)
    return lib.kda_prefill_split(dtype, B, T, H, dk, dv, chunk, P, p["q"], p["k"], p["v"],
                                 p["z"], p["beta"], p["A"], p["S0"], p["o"], p["S_T"], p["ws"],
                                 ws_bytes, None)


P_ = P


def test_split_argument_errors(lib):
    assert split(lib, T=-1) == SHAPE
    assert split(lib, P=0) == UNSUP
    assert split(lib, P=1025) == UNSUP
    assert split(lib, dtype=F32) == UNSUP            # the role-split kernel only
    assert split(lib, chunk=32) == UNSUP
    assert split(lib, dk=16, dv=16) == UNSUP
    assert split(lib, ptrs={"z": None}) == NULL
    assert split(lib, ptrs={"ws": None}) == WORKSPACE
    assert split(lib, ws_bytes=4096) == WORKSPACE
    assert split(lib, ptrs={"ws": P_(9, 8)}) == MISALIGNED
    assert split(lib, ptrs={"ws": P_(7, 0)}) == ALIAS   # workspace over o
    assert split(lib, ptrs={"o": P_(0, 64)}) == ALIAS   # the plain call's rules hold
    assert split(lib, B=0) == OK
    # workspace: three [B*P, H, d, d] fp32 state sets plus offsets
    n = lib.kda_prefill_split_workspace_size(BF16, 1, 4096, 2, 128, 128, 16, 4)
    assert n >= 3 * 4 * 2 * 128 * 128 * 4
    assert lib.kda_prefill_split_workspace_size(BF16, 1, 4096, 2, 128, 128, 16, 1) == 0
    assert lib.kda_prefill_split_workspace_size(F32, 1, 4096, 2, 128, 128, 16, 4) == 0
    assert lib.kda_prefill_split_workspace_size(BF16, 1, 4096, 2, 128, 128, 64, 4) == n
    assert lib.kda_prefill_split_workspace_size(BF16, 1, 4096, 2, 128, 128, 32, 4) == 0
    assert split(lib, chunk=64, ptrs={"ws": None}) == WORKSPACE
    assert split(lib, chunk=64, B=0) == OK


def conv_varlen(lib, dtype=BF16, N=3, T=64, H=2, dk=128, dv=128, conv=None, sin=None,
                sout=None, ptrs=None):
    p = {n: P(i) for i, n in enumerate(["q", "k", "v", "qo", "ko", "vo", "cu"])}
    if ptrs:
        p.update(ptrs)
    cs = conv if conv is not None else short_conv()
    return lib.kda_conv_norm_varlen(dtype, N, T, H, dk, dv, p["cu"], ctypes.byref(cs), p["q"],
                                    p["k"], p["v"], sin, sout, p["qo"], p["ko"], p["vo"], None)


def test_conv_norm_varlen_argument_errors(lib):
    assert conv_varlen(lib, N=-1) == SHAPE
    assert conv_varlen(lib, dk=64, dv=64) == UNSUP
    assert conv_varlen(lib, conv=short_conv(W=6)) == UNSUP
    assert conv_varlen(lib, ptrs={"cu": None}) == NULL            # N > 0 needs offsets
    assert conv_varlen(lib, ptrs={"cu": P(6, 4)}) == MISALIGNED   # int64 offsets
    assert conv_varlen(lib, ptrs={"qo": P(6, 0)}) == ALIAS        # output over the offsets
    assert conv_varlen(lib, ptrs={"vo": P(2, 32)}) == ALIAS       # output over v
    assert conv_varlen(lib, sin=states(50, 51, 52), sout=states(53, 52, 55)) == ALIAS
    assert conv_varlen(lib, N=0, ptrs={"cu": None}) == OK


# ------------------------------------------------------------- backward ----

BWD_NAMES = ["q", "k", "v", "z", "beta", "A", "S0", "dO", "dST", "dq", "dk", "dv", "dz",
             "dbeta", "dA", "dS0", "ws"]


def bwd(lib, dtype=BF16, B=1, T=40, H=2, dk=128, dv=128, ptrs=None, ws_bytes=None):
    p = {n: P(i) for i, n in enumerate(BWD_NAMES)}
    if ptrs:
        p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.kda_prefill_bwd_workspace_size(dtype, B, T, H, dk, dv)
    return lib.kda_prefill_bwd(dtype, B, T, H, dk, dv, *(p[n] for n in BWD_NAMES[:-1]),
                               p["ws"], ws_bytes, None)


def test_backward_argument_errors(lib):
    assert bwd(lib, T=-1) == SHAPE
    assert bwd(lib, B=1, T=1, H=1 << 17, ws_bytes=1 << 40) == SHAPE   # 64-token tile past 2^31 bytes
    assert bwd(lib, dtype=7) == UNSUP
    assert bwd(lib, dk=64, dv=64) == UNSUP
    assert bwd(lib, dk=128, dv=16) == UNSUP
    for name in ("q", "beta", "dO", "dq", "dbeta", "dA", "dS0", "A"):
        assert bwd(lib, ptrs={name: None}) == NULL, name
    assert bwd(lib, ptrs={"ws": None}) == WORKSPACE
    assert bwd(lib, ws_bytes=256) == WORKSPACE
    assert bwd(lib, ptrs={"dz": P(12, 4)}) == MISALIGNED
    assert bwd(lib, ptrs={"dq": P(1, 64)}) == ALIAS        # a gradient over k
    assert bwd(lib, ptrs={"dk": P(9, 16)}) == ALIAS        # two gradients overlap
    assert bwd(lib, ptrs={"ws": P(0, 0)}) == ALIAS         # workspace over q
    assert bwd(lib, ptrs={"dS0": P(6, 0)}) == ALIAS        # dS0 over S0
    assert bwd(lib, H=0) == OK                              # nothing to do
    # a dispatch counts work-items in 32 bits: at most 2^32 / 1024 chunk-heads
    assert bwd(lib, B=1, T=16 * 4096, H=1024, ws_bytes=1 << 62) == SHAPE
    # S0 and dS_T are optional
    assert lib.kda_prefill_bwd_workspace_size(F32, 1, 40, 2, 16, 16) > 0
    assert lib.kda_prefill_bwd_workspace_size(BF16, 1, 40, 2, 64, 64) == 0


def test_backward_workspace_holds_forward_and_checkpoints(lib):
    B, T, H, d = 2, 100, 3, 128
    # fp32: the rerun forward's o, fp32 checkpoints and final states
    n = lib.kda_prefill_bwd_workspace_size(F32, B, T, H, d, d)
    o = B * T * H * d * 4
    ckpt = B * (T // 16) * H * d * d * 4
    assert n >= o + ckpt + B * H * d * d * 4
    # bf16 (matrix-core backward): states only, checkpoints in bf16, plus the
    # per-chunk dS' hand-off (d*d bf16 per chunk)
    n = lib.kda_prefill_bwd_workspace_size(BF16, B, T, H, d, d)
    units = B * H * ((T + 15) // 16)
    assert n >= ckpt // 2 + B * H * d * d * 4 + units * d * d * 2


def test_noalloc_varlen_validates_before_any_device_call(lib):
    """kda_prefill_varlen_noalloc checks its arguments before it touches the
    device (its scratch is looked up only for a valid call), so these statuses
    come back without a GPU."""
    i64 = ctypes.c_int64
    f = lib.kda_prefill_varlen_noalloc
    cu = P(20)

    def call(dtype=BF16, N=3, T=64, H=2, d=128, chunk=16, cu_=cu, beta=P(5)):
        return f(dtype, N, T, H, d, d, chunk, cu_, P(1), P(2), P(3), P(4), beta, P(6), None,
                 P(8), P(9), 0, None, 0, None, 0)
    assert call(N=8193) == 6                    # beyond the static scratch
    assert call(dtype=7) == 3
    assert call(d=64) == 3
    assert call(chunk=32) == 3
    assert call(N=-1) == 2
    assert call(cu_=None) == 1
    assert call(beta=None) == 1
    assert call(beta=ctypes.c_void_p(BASE + 8)) == 4
