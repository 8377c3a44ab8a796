"""GPU parity of the packed variable-length prefill and its state checkpoints.

Each packed sequence must give what the oracle gives for that sequence alone
(its own initial state, the same seeded inputs); checkpoint j of a sequence is
the oracle's state after its first j*ckpt_every tokens (the state carry of
the recurrence, pinned on the oracle side by the split-sequence invariant).
Tolerances as in test_gpu_parity: 1e-4 (fp32), 2e-2 (bf16), normwise per
head slice.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_attention_chunkwise_amd.inputs import WORKLOADS, make_varlen_inputs
from tests.gpu_helpers import TOL, diag, host, slice_relerr, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import linear_recurrent_attention_chunkwise_amd as m
    assert m.abi_version() == 8
    return m


def _say(*a):
    print(*a, flush=True)


def _seq(inp, cu, i):
    """Host arrays of sequence i as a dense batch of one."""
    a, b = int(cu[i]), int(cu[i + 1])
    d = {n: host(inp[n][a:b])[None] for n in ("q", "k", "v", "z", "beta")}
    d["A"] = host(inp["A"])
    d["S0"] = host(inp["S0"][i:i + 1])
    return d


def _oracle_seq(inp, cu, i, T=None):
    d = _seq(inp, cu, i)
    if T is not None:
        for n in ("q", "k", "v", "z", "beta"):
            d[n] = d[n][:, :T]
    return oracle.prefill(d["q"], d["k"], d["v"], d["z"], d["beta"], d["A"], d["S0"])


def _run(kda, inp, dev, chunk, every=0, dvb=0):
    g = to_dev(inp, dev)
    o, S_T, ck = kda.prefill_varlen(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"],
                                    inp["cu_seqlens"], S0=g["S0"], chunk=chunk,
                                    ckpt_every=every, dv_per_block=dvb)
    torch.cuda.synchronize()
    return o, S_T, ck


def _compare_sequences(kda, dev, w, lengths, chunk, dvb=0):
    inp = make_varlen_inputs(w, lengths)
    cu = inp["cu_seqlens"].tolist()
    _say(f"[varlen] {w.dtype} d={w.dk} H={w.H} lengths={lengths} chunk={chunk} dvb={dvb}")
    o, S_T, _ = _run(kda, inp, dev, chunk, dvb=dvb)
    tol = TOL[inp["q"].dtype]
    for i in range(len(lengths)):
        o_ref, S_ref = _oracle_seq(inp, cu, i)
        a, b = cu[i], cu[i + 1]
        es = slice_relerr(host(S_T[i:i + 1]), S_ref, 1)
        eo = slice_relerr(host(o[a:b])[None], o_ref, 2) if b > a else 0.0
        _say(f"   seq {i} len {b - a}: o err {eo:.2e} S_T err {es:.2e}")
        assert eo <= tol and es <= tol, (i, eo, es)


@pytest.mark.parametrize("chunk", [16, 64])
def test_varlen_bf16_d128(kda, gpu_device, chunk):
    w = WORKLOADS["k3_prefill_bf16"].with_(H=4)
    _compare_sequences(kda, gpu_device, w, [37, 0, 16, 1, 100, 64, 5], chunk)


def test_varlen_bf16_d128_column_splits(kda, gpu_device):
    w = WORKLOADS["k3_prefill_bf16"].with_(H=2, seed=11)
    for dvb in (32, 128):
        _compare_sequences(kda, gpu_device, w, [45, 3, 80], 16, dvb=dvb)


@pytest.mark.parametrize("chunk", [16, 64])
def test_varlen_fp32_d16(kda, gpu_device, chunk):
    w = WORKLOADS["tiny_prefill_f32"].with_(H=3, s0_std=0.5)
    _compare_sequences(kda, gpu_device, w, [5, 17, 0, 33, 64], chunk)


@pytest.mark.parametrize("chunk,every,dvb", [(16, 16, 0), (16, 48, 0), (16, 32, 32),
                                            (16, 32, 128), (64, 64, 0), (64, 128, 32),
                                            (64, 64, 64)])
def test_varlen_checkpoints(kda, gpu_device, chunk, every, dvb):
    w = WORKLOADS["k3_prefill_bf16"].with_(H=3, seed=12)
    lengths = [70, 130, 31, 0, 64]
    inp = make_varlen_inputs(w, lengths)
    cu = inp["cu_seqlens"].tolist()
    _say(f"[ckpt] lengths={lengths} chunk={chunk} every={every}")
    o, S_T, ck = _run(kda, inp, gpu_device, chunk, every=every, dvb=dvb)
    rows, total = kda.checkpoint_rows(lengths, every)
    assert ck.shape[0] == total == sum(L // every for L in lengths)
    tol = TOL[inp["q"].dtype]
    for i, L in enumerate(lengths):
        o_ref, S_ref = _oracle_seq(inp, cu, i)
        a, b = cu[i], cu[i + 1]
        assert slice_relerr(host(S_T[i:i + 1]), S_ref, 1) <= tol
        if b > a:   # outputs too: a checkpointing build must not disturb them
            assert slice_relerr(host(o[a:b])[None], o_ref, 2) <= tol
        for j in range(1, L // every + 1):
            _, S_ref = _oracle_seq(inp, cu, i, T=j * every)
            e = slice_relerr(host(ck[rows[i] + j - 1:rows[i] + j]), S_ref, 1)
            _say(f"   seq {i} checkpoint {j} (after {j * every} tokens): err {e:.2e}")
            assert e <= tol, (i, j, e)


@pytest.mark.parametrize("chunk,dvb", [(16, 0), (64, 0), (64, 16)])
def test_varlen_checkpoints_fp32_d16(kda, gpu_device, chunk, dvb):
    w = WORKLOADS["tiny_prefill_f32"].with_(H=2, s0_std=0.5, seed=16)
    lengths = [130, 0, 64, 70]
    inp = make_varlen_inputs(w, lengths)
    cu = inp["cu_seqlens"].tolist()
    o, S_T, ck = _run(kda, inp, gpu_device, chunk, every=64, dvb=dvb)
    rows, _ = kda.checkpoint_rows(lengths, 64)
    tol = TOL[inp["q"].dtype]
    for i, L in enumerate(lengths):
        o_ref, S_ref = _oracle_seq(inp, cu, i)
        a, b = cu[i], cu[i + 1]
        assert slice_relerr(host(S_T[i:i + 1]), S_ref, 1) <= tol
        if b > a:
            assert slice_relerr(host(o[a:b])[None], o_ref, 2) <= tol
        for j in range(1, L // 64 + 1):
            _, S_j = _oracle_seq(inp, cu, i, T=64 * j)
            e = slice_relerr(host(ck[rows[i] + j - 1:rows[i] + j]), S_j, 1)
            _say(f"   seq {i} checkpoint {j}: err {e:.2e}")
            assert e <= tol


def test_varlen_checkpoints_chunk64_full_shape(kda, gpu_device):
    """bf16, dk = 128, 64-token chunks, 64 value columns per workgroup, with
    checkpoints, on the K3 head count: the outputs (not only the states) of
    every sequence against the oracle.  This build once returned wrong
    outputs with right states: an MFMA product of the 16x16x16 shape summed
    directly onto a fresh 16x16x32 result, which the compiler does not
    separate by the wait states the hardware needs."""
    w = WORKLOADS["k3_prefill_bf16"]
    lengths = [1024, 333, 64, 2048]
    inp = make_varlen_inputs(w, lengths)
    cu = inp["cu_seqlens"].tolist()
    _say(f"[ckpt] K3 heads, lengths={lengths} chunk=64 every=256 dvb=64")
    o, S_T, ck = _run(kda, inp, gpu_device, 64, every=256, dvb=64)
    o0, S0_, _ = _run(kda, inp, gpu_device, 64, dvb=64)
    # the checkpointing build must not change the outputs beyond rounding order
    assert slice_relerr(host(o)[None], host(o0)[None], 2) <= 1e-6
    assert slice_relerr(host(S_T), host(S0_), 1) <= 1e-6
    rows, _ = kda.checkpoint_rows(lengths, 256)
    for i in (0, 3):
        o_ref, S_ref = _oracle_seq(inp, cu, i)
        a, b = cu[i], cu[i + 1]
        eo = slice_relerr(host(o[a:b])[None], o_ref, 2)
        es = slice_relerr(host(S_T[i:i + 1]), S_ref, 1)
        _, S_1 = _oracle_seq(inp, cu, i, T=256)
        ec = slice_relerr(host(ck[rows[i]:rows[i] + 1]), S_1, 1)
        _say(f"   seq {i}: o err {eo:.2e}  S_T err {es:.2e}  first checkpoint err {ec:.2e}")
        assert eo <= 2e-2 and es <= 2e-2 and ec <= 2e-2


def test_varlen_bench_workload(kda, gpu_device):
    """The packed workload the bench times (eight sequences of lengths 4096,
    1000, 37, 2500, 16, 513, 64, 3000; all 96 heads; 16-token chunks; a
    checkpoint every 1024 tokens), every head of every sequence and every
    checkpoint against the oracle."""
    lengths, every = [4096, 1000, 37, 2500, 16, 513, 64, 3000], 1024
    w = WORKLOADS["k3_prefill_bf16"].with_(seed=5)
    inp = make_varlen_inputs(w, lengths)
    cu = inp["cu_seqlens"].tolist()
    _say(f"[varlen] bench workload H={w.H} lengths={lengths} every={every}")
    o, S_T, ck = _run(kda, inp, gpu_device, 16, every=every)
    rows, _ = kda.checkpoint_rows(lengths, every)
    worst = 0.0
    for i, L in enumerate(lengths):
        o_ref, S_ref = _oracle_seq(inp, cu, i)
        a, b = cu[i], cu[i + 1]
        eo = slice_relerr(host(o[a:b])[None], o_ref, 2)
        es = slice_relerr(host(S_T[i:i + 1]), S_ref, 1)
        ec = 0.0
        for j in range(1, L // every + 1):
            _, S_j = _oracle_seq(inp, cu, i, T=j * every)
            ec = max(ec, slice_relerr(host(ck[rows[i] + j - 1:rows[i] + j]), S_j, 1))
        _say(f"   seq {i} len {L}: o err {eo:.2e}  S_T err {es:.2e}  checkpoints err {ec:.2e}"
             f"  (o {diag(host(o[a:b])[None], o_ref)})")
        worst = max(worst, eo, es, ec)
    _say(f"   worst over outputs, final states and {ck.shape[0]} checkpoints: {worst:.2e}")
    assert worst <= TOL[inp["q"].dtype]


def test_varlen_equals_dense_bitwise(kda, gpu_device):
    w = WORKLOADS["k3_prefill_bf16"].with_(H=4, seed=13)
    N, L = 3, 50
    inp = make_varlen_inputs(w, [L] * N)
    o, S_T, _ = _run(kda, inp, gpu_device, 16)
    g = to_dev(inp, gpu_device)
    dense = {n: g[n].reshape((N, L) + tuple(g[n].shape[1:])) for n in ("q", "k", "v", "z", "beta")}
    od, Sd = kda.prefill(dense["q"], dense["k"], dense["v"], dense["z"], dense["beta"], g["A"],
                         g["S0"], chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(od.shape), od)
    assert torch.equal(S_T, Sd)


def test_resume_from_checkpoint_bitwise(kda, gpu_device):
    """Continuing from a checkpoint reproduces the uninterrupted run exactly:
    the checkpoint is the exact fp32 state and chunk boundaries line up."""
    w = WORKLOADS["k3_prefill_bf16"].with_(H=2, seed=14)
    L, every = 100, 32
    inp = make_varlen_inputs(w, [L])
    o, S_T, ck = _run(kda, inp, gpu_device, 16, every=every)
    g = to_dev(inp, gpu_device)
    t0 = 2 * every
    tail = {n: g[n][t0:].unsqueeze(0).contiguous() for n in ("q", "k", "v", "z", "beta")}
    S_mid = ck[1:2].clone()
    ot, St = kda.prefill(tail["q"], tail["k"], tail["v"], tail["z"], tail["beta"], g["A"],
                         S_mid, chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(ot[0], o[t0:])
    assert torch.equal(St, S_T)


def test_malformed_offsets_are_clamped(kda, gpu_device):
    """Offsets outside [0, T] are clamped by the kernels (no access outside the
    tensors): [0, 5, 10**6] over T = 20 acts as [0, 5, 20], and a negative
    offset as 0."""
    w = WORKLOADS["k3_prefill_bf16"].with_(H=2, seed=15)
    inp = make_varlen_inputs(w, [5, 15])
    g = to_dev(inp, gpu_device)
    lib = kda.kda._load()
    T, H, d = g["q"].shape

    def raw(cu_list):
        cu = torch.tensor(cu_list, dtype=torch.int64, device=gpu_device)
        o = torch.zeros((T, H, d), dtype=g["q"].dtype, device=gpu_device)
        S = torch.zeros((2, H, d, d), dtype=torch.float32, device=gpu_device)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        ws_bytes = lib.kda_prefill_varlen_workspace_size(2)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=gpu_device)
        st = lib.kda_prefill_varlen(1, 2, T, H, d, d, 16, p(cu), p(g["q"]), p(g["k"]), p(g["v"]),
                                    p(g["z"]), p(g["beta"]), p(g["A"]), p(g["S0"]), p(o), p(S),
                                    0, None, 0, p(ws), ws_bytes, None, 0)
        torch.cuda.synchronize()
        assert st == 0
        return o, S

    o_ok, S_ok = raw([0, 5, 20])
    o_big, S_big = raw([0, 5, 10 ** 6])
    assert torch.equal(o_ok, o_big) and torch.equal(S_ok, S_big)
    o_neg, S_neg = raw([0, -7, 20])     # sequence 0 empty, sequence 1 = all 20 tokens
    S0 = g["S0"]
    assert torch.equal(S_neg[0], S0[0])


def test_longest_first_order_does_not_change_results(kda, gpu_device):
    """Sequences are dispatched longest first; a sequence's result does not
    depend on where it sits in the packing (bitwise)."""
    w = WORKLOADS["k3_prefill_bf16"].with_(H=2, seed=18)
    lengths = [5, 300, 40, 300, 0, 129]
    inp = make_varlen_inputs(w, lengths)
    cu = inp["cu_seqlens"].tolist()
    o, S_T, _ = _run(kda, inp, gpu_device, 16)
    perm = [5, 2, 0, 4, 3, 1]
    pieces = {n: [inp[n][cu[i]:cu[i + 1]] for i in perm] for n in ("q", "k", "v", "z", "beta")}
    inp2 = {n: torch.cat(pieces[n]) for n in pieces}
    inp2["A"] = inp["A"]
    inp2["S0"] = inp["S0"][perm].contiguous()
    lens2 = [lengths[i] for i in perm]
    inp2["cu_seqlens"] = torch.tensor([0] + list(np.cumsum(lens2)), dtype=torch.int64)
    o2, S2, _ = _run(kda, inp2, gpu_device, 16)
    cu2 = inp2["cu_seqlens"].tolist()
    for pos, i in enumerate(perm):
        assert torch.equal(S2[pos], S_T[i])
        assert torch.equal(o2[cu2[pos]:cu2[pos + 1]], o[cu[i]:cu[i + 1]])
