"""GPU parity of the layer prologue (short causal convolutions, optional SiLU,
q/k L2 normalization) and of the entry points that run it ahead of the
recurrence, against the fp64 oracle of ``oracle/prologue.py``.

Tolerances are those of the recurrence (normwise per (b, h) slice): 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs.  Convolution states hold raw inputs and are
compared exactly.  Cases cover every width 1..4, both activations, fresh and
continued sequences, empty and ragged segments, head counts that leave lanes
of a wave idle, and the K3 shapes at full size.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import prologue
from linear_recurrent_attention_chunkwise_amd.inputs import (WORKLOADS, make_layer_decode_inputs,
                                                             make_layer_inputs)
from tests.gpu_helpers import TOL, host, slice_relerr

pytestmark = pytest.mark.gpu

ACTS = ("none", "silu")
EPS = 1e-6


@pytest.fixture(scope="module")
def kda():
    import linear_recurrent_attention_chunkwise_amd as m
    assert m.abi_version() == 8
    return m


def _say(*a):
    print(*a, flush=True)


def _dev(inp, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _states(g, use):
    return (g["sq"], g["sk"], g["sv"]) if use else None


def _host_states(inp, use):
    return tuple(host(inp[n]) for n in ("sq", "sk", "sv")) if use else (None, None, None)


def _check_states(got, ref, W):
    for a, b in zip(got, ref):
        assert tuple(a.shape)[1] == W - 1
        assert np.array_equal(host(a), b), "convolution state differs"


# ------------------------------------------------------------ kda_conv_norm ----

CONV_CASES = [(wname, W, act, st)
              for wname in ("k3_prefill_bf16", "tiny_prefill_f32")
              for W in (1, 2, 3, 4) for act in ACTS for st in (False, True)]


@pytest.mark.parametrize("wname,W,act,use_state", CONV_CASES)
def test_conv_norm_matches_oracle(kda, gpu_device, wname, W, act, use_state):
    w = WORKLOADS[wname].with_(B=2, H=3, s0_std=None)
    for T in (0, 1, 2, 5, 17, 40):
        _say(f"[conv_norm] {wname} W={W} act={act} state={use_state} T={T}")
        inp = make_layer_inputs(w, W, T=T)
        g = _dev(inp, gpu_device)
        qh, kh, vc, ns = kda.conv_norm(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["wv"],
                                       state=_states(g, use_state), act=act, eps=EPS)
        torch.cuda.synchronize()
        sq, sk, sv = _host_states(inp, use_state)
        rq, rk, rv, rs = prologue.conv_norm(host(inp["q"]), host(inp["k"]), host(inp["v"]),
                                            host(inp["wq"]), host(inp["wk"]), host(inp["wv"]),
                                            sq, sk, sv, act, EPS)
        tol = TOL[inp["q"].dtype]
        if T > 0:
            errs = [slice_relerr(host(x), r, 2) for x, r in ((qh, rq), (kh, rk), (vc, rv))]
            assert max(errs) <= tol, errs
        _check_states(ns, rs, W)


def test_conv_norm_k3_full_size(kda, gpu_device):
    """K3 prefill shape (B=1, H=96, T=4096, bf16), width 4, SiLU, continued
    sequence: every output element against the oracle."""
    w = WORKLOADS["k3_prefill_bf16"]
    inp = make_layer_inputs(w, 4)
    _say(f"[conv_norm] {w.name} full size")
    g = _dev(inp, gpu_device)
    qh, kh, vc, ns = kda.conv_norm(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["wv"],
                                   state=_states(g, True), act="silu", eps=EPS)
    torch.cuda.synchronize()
    rq, rk, rv, rs = prologue.conv_norm(host(inp["q"]), host(inp["k"]), host(inp["v"]),
                                        host(inp["wq"]), host(inp["wk"]), host(inp["wv"]),
                                        *_host_states(inp, True), "silu", EPS)
    errs = [slice_relerr(host(x), r, 2) for x, r in ((qh, rq), (kh, rk), (vc, rv))]
    _say(f"   errors {errs}")
    assert max(errs) <= TOL[torch.bfloat16]
    _check_states(ns, rs, 4)
    # the normalized rows have unit norm up to bf16 rounding
    n = torch.linalg.vector_norm(qh.float(), dim=-1)
    assert torch.max(torch.abs(n - 1)).item() < 1e-2


def test_conv_norm_segments_carry_exactly(kda, gpu_device):
    """Two segments with the state carried give the same bits as one segment."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=2, H=2)
    inp = _dev(make_layer_inputs(w, 4, T=70), gpu_device)
    whole = kda.conv_norm(inp["q"], inp["k"], inp["v"], inp["wq"], inp["wk"], inp["wv"],
                          state=_states(inp, True), act="silu")
    parts, st = [], _states(inp, True)
    for lo, hi in ((0, 1), (1, 33), (33, 70)):
        seg = [inp[n][:, lo:hi].contiguous() for n in ("q", "k", "v")]
        r = kda.conv_norm(*seg, inp["wq"], inp["wk"], inp["wv"], state=st, act="silu")
        parts.append(r[:3])
        st = r[3]
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(torch.cat([p[i] for p in parts], dim=1), whole[i])
    for a, b in zip(st, whole[3]):
        assert torch.equal(a, b)


# ----------------------------------------------------- kda_conv_norm_varlen ----

VARLEN_CONV_LENGTHS = [0, 1, 2, 5, 17, 40, 3, 100, 0, 33]


@pytest.mark.parametrize("wname", ["k3_prefill_bf16", "tiny_prefill_f32"])
@pytest.mark.parametrize("W,act", [(4, "silu"), (2, "none"), (1, "silu")])
@pytest.mark.parametrize("use_state", [False, True])
def test_conv_norm_varlen_equals_per_sequence(kda, gpu_device, wname, W, act, use_state):
    """Packed sequences give, sequence by sequence, the bits of kda_conv_norm on
    that sequence alone: taps never cross a sequence boundary, each sequence
    reads its own state rows, and every new state (empty and short sequences
    included) is that sequence's."""
    lengths = VARLEN_CONV_LENGTHS
    Tt = sum(lengths)
    N = len(lengths)
    w = WORKLOADS[wname].with_(B=1, H=3)
    inp = make_layer_inputs(w.with_(B=N), W, T=max(lengths))
    # packed tokens: sequence i takes its first lengths[i] tokens of batch row i
    pk = {n: torch.cat([inp[n][i, :L] for i, L in enumerate(lengths)], dim=0).contiguous()
          for n in ("q", "k", "v")}
    g = {n: pk[n].to(gpu_device) for n in pk}
    taps = tuple(inp[n].to(gpu_device) for n in ("wq", "wk", "wv"))
    st = tuple(inp[n].to(gpu_device) for n in ("sq", "sk", "sv")) if use_state else None
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int64)
    _say(f"[conv_norm_varlen] {wname} W={W} act={act} state={use_state} lengths={lengths}")
    qh, kh, vc, ns = kda.conv_norm_varlen(g["q"], g["k"], g["v"], *taps, cu, state=st, act=act,
                                          eps=EPS)
    torch.cuda.synchronize()
    off = 0
    for i, L in enumerate(lengths):
        seg = [x[off:off + L].unsqueeze(0).contiguous() for x in (g["q"], g["k"], g["v"])]
        sti = tuple(t[i:i + 1].contiguous() for t in st) if use_state else None
        r = kda.conv_norm(*seg, *taps, state=sti, act=act, eps=EPS)
        torch.cuda.synchronize()
        for a, b_ in zip((qh, kh, vc), r[:3]):
            assert torch.equal(a[off:off + L], b_[0]), (i, L)
        for a, b_ in zip(ns, r[3]):
            assert torch.equal(a[i:i + 1], b_), (i, L)
        off += L
    # and the oracle on the whole packing, sequence by sequence
    tol = TOL[inp["q"].dtype]
    off = 0
    for i, L in enumerate(lengths):
        sti = tuple(host(inp[n][i:i + 1]) for n in ("sq", "sk", "sv")) if use_state else (
            None, None, None)
        rq, rk, rv, rs = prologue.conv_norm(*(host(pk[n][off:off + L]).reshape(
                                                  1, L, 3, pk[n].shape[-1])
                                              for n in ("q", "k", "v")),
                                            host(inp["wq"]), host(inp["wk"]), host(inp["wv"]),
                                            *sti, act, EPS)
        if L > 0:
            errs = [slice_relerr(host(x[off:off + L])[None], r_, 2)
                    for x, r_ in ((qh, rq), (kh, rk), (vc, rv))]
            assert max(errs) <= tol, (i, errs)
        for a, b_ in zip(ns, rs):
            assert np.array_equal(host(a[i:i + 1]), b_), i
        off += L


# --------------------------------------------------------- kda_prefill_conv ----

def _oracle_layer(inp, W, act, use_state, S0=None):
    sq, sk, sv = _host_states(inp, use_state)
    st = (sq, sk, sv) if use_state else None
    return oracle.prefill_conv(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["z"]),
                               host(inp["beta"]), host(inp["A"]), host(inp["wq"]),
                               host(inp["wk"]), host(inp["wv"]), st, act, EPS,
                               host(inp["S0"]) if S0 is None else S0)


PREFILL_CASES = [("k3_prefill_bf16", 16), ("k3_prefill_bf16", 64),
                 ("tiny_prefill_f32", 16), ("tiny_prefill_f32", 64)]


@pytest.mark.parametrize("wname,chunk", PREFILL_CASES)
@pytest.mark.parametrize("W,act,use_state", [(4, "silu", True), (2, "none", False),
                                             (1, "silu", False)])
def test_prefill_conv_matches_oracle(kda, gpu_device, wname, chunk, W, act, use_state):
    w = WORKLOADS[wname].with_(B=2, H=2, s0_std=0.5)
    for T in (1, 37, 100):
        _say(f"[prefill_conv] {wname} chunk={chunk} W={W} act={act} state={use_state} T={T}")
        inp = make_layer_inputs(w, W, T=T)
        g = _dev(inp, gpu_device)
        o, S_T, ns = kda.prefill_conv(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"],
                                      g["wq"], g["wk"], g["wv"], state=_states(g, use_state),
                                      act=act, eps=EPS, S0=g["S0"], chunk=chunk)
        torch.cuda.synchronize()
        o_ref, S_ref, st_ref = _oracle_layer(inp, W, act, use_state)
        tol = TOL[inp["q"].dtype]
        eo, es = slice_relerr(host(o), o_ref, 2), slice_relerr(host(S_T), S_ref, 1)
        _say(f"   o err {eo:.3e}  S_T err {es:.3e}")
        assert eo <= tol and es <= tol
        _check_states(ns, st_ref, W)


def test_prefill_conv_is_conv_norm_then_prefill(kda, gpu_device):
    """The composite entry point gives the bits of its two steps run apart."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=2, H=3)
    g = _dev(make_layer_inputs(w, 4, T=150), gpu_device)
    o, S_T, ns = kda.prefill_conv(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], g["wq"],
                                  g["wk"], g["wv"], state=_states(g, True), act="silu",
                                  S0=g["S0"])
    qh, kh, vc, ns2 = kda.conv_norm(g["q"], g["k"], g["v"], g["wq"], g["wk"], g["wv"],
                                    state=_states(g, True), act="silu")
    o2, S2 = kda.prefill(qh, kh, vc, g["z"], g["beta"], g["A"], g["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S_T, S2)
    for a, b in zip(ns, ns2):
        assert torch.equal(a, b)


def test_prefill_conv_segments_carry(kda, gpu_device):
    """A sequence prefilled in two calls (both states carried, split on a chunk
    boundary) gives the bits of one call."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=2, H=2)
    g = _dev(make_layer_inputs(w, 4, T=96), gpu_device)
    o, S_T, ns = kda.prefill_conv(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], g["wq"],
                                  g["wk"], g["wv"], state=_states(g, True), act="silu",
                                  S0=g["S0"])
    cut = 48
    part = {n: (g[n][:, :cut].contiguous(), g[n][:, cut:].contiguous())
            for n in ("q", "k", "v", "z", "beta")}
    o1, S1, st1 = kda.prefill_conv(*(part[n][0] for n in ("q", "k", "v", "z", "beta")), g["A"],
                                   g["wq"], g["wk"], g["wv"], state=_states(g, True),
                                   act="silu", S0=g["S0"])
    o2, S2, st2 = kda.prefill_conv(*(part[n][1] for n in ("q", "k", "v", "z", "beta")), g["A"],
                                   g["wq"], g["wk"], g["wv"], state=st1, act="silu", S0=S1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], dim=1), o) and torch.equal(S2, S_T)
    for a, b in zip(st2, ns):
        assert torch.equal(a, b)


def test_prefill_conv_k3_sampled_heads(kda, gpu_device):
    """K3 prefill shape at full size (B=1, H=96, T=4096, bf16, chunk 16, the
    launch bench.py times); the oracle runs heads 0, 47 and 95."""
    w = WORKLOADS["k3_prefill_bf16"]
    W, act = 4, "silu"
    inp = make_layer_inputs(w, W)
    _say(f"[prefill_conv] {w.name} full size, oracle on heads 0, 47, 95")
    g = _dev(inp, gpu_device)
    o, S_T, ns = kda.prefill_conv(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], g["wq"],
                                  g["wk"], g["wv"], state=_states(g, True), act=act,
                                  S0=g["S0"])
    torch.cuda.synchronize()
    heads = [0, 47, 95]
    sub = {n: inp[n][:, :, heads].contiguous() for n in ("q", "k", "v", "z", "beta")}
    for n in ("sq", "sk", "sv"):
        sub[n] = inp[n][:, :, heads].contiguous()
    for n in ("wq", "wk", "wv"):
        sub[n] = inp[n][heads].contiguous()
    sub["A"] = inp["A"][heads]
    sub["S0"] = inp["S0"][:, heads].contiguous()
    o_ref, S_ref, st_ref = _oracle_layer(sub, W, act, True)
    eo = slice_relerr(host(o[:, :, heads]), o_ref, 2)
    es = slice_relerr(host(S_T[:, heads]), S_ref, 1)
    _say(f"   o err {eo:.3e}  S_T err {es:.3e}")
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]
    for a, b in zip(ns, st_ref):
        assert np.array_equal(host(a[:, :, heads]), b)


# ----------------------------------------------------- kda_decode_step_conv ----

DECODE_CASES = [(wname, W, act) for wname in ("k3_decode_bf16", "tiny_decode_f32")
                for W in (1, 2, 3, 4) for act in ACTS]


def _decode_workload(wname):
    if wname == "tiny_decode_f32":
        return WORKLOADS["k3_decode_bf16"].with_(name=wname, dk=16, dv=16, dtype="f32")
    return WORKLOADS[wname]


@pytest.mark.parametrize("wname,W,act", DECODE_CASES)
def test_decode_conv_matches_oracle(kda, gpu_device, wname, W, act):
    w = _decode_workload(wname).with_(B=3, H=2)
    steps = 6
    inp = make_layer_decode_inputs(w, W, steps=steps)
    _say(f"[decode_conv] {wname} W={W} act={act} steps={steps}")
    g = _dev(inp, gpu_device)
    rng = np.random.default_rng(7)
    S0 = rng.standard_normal(tuple(inp["S"].shape)) * 0.1
    S = torch.tensor(S0, dtype=torch.float32, device=gpu_device)
    st = tuple(t.clone() for t in _states(g, True))
    S_ref, st_ref = S0, _host_states(inp, True)
    tol = TOL[inp["q"].dtype]
    for t in range(steps):
        # per-step copies: a step's slice of [steps, B, H] need not be 16-byte aligned
        step = [g[n][t].clone() for n in ("q", "k", "v", "z", "beta")]
        o = kda.decode_step_conv(*step, g["A"], g["wq"], g["wk"], g["wv"], st, S, act=act,
                                 eps=EPS)
        torch.cuda.synchronize()
        o_ref, S_ref, st_ref = oracle.decode_step_conv(
            host(inp["q"][t]), host(inp["k"][t]), host(inp["v"][t]), host(inp["z"][t]),
            host(inp["beta"][t]), host(inp["A"]), host(inp["wq"]), host(inp["wk"]),
            host(inp["wv"]), st_ref, S_ref, act, EPS)
        eo = slice_relerr(host(o)[:, None], o_ref[:, None], 2)
        assert eo <= tol, (t, eo)
        _check_states(st, st_ref, W)
    es = slice_relerr(host(S), S_ref, 1)
    _say(f"   final S err {es:.3e}")
    assert es <= tol


def test_decode_conv_continues_prefill_conv(kda, gpu_device):
    """Prefill of T tokens, then single decode steps, matches the oracle's one
    prefill over all tokens (states handed from prefill to decode)."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=2, H=2, s0_std=0.5)
    T, extra, W, act = 45, 4, 4, "silu"
    inp = make_layer_inputs(w, W, T=T + extra)
    g = _dev(inp, gpu_device)
    head = {n: g[n][:, :T].contiguous() for n in ("q", "k", "v", "z", "beta")}
    o, S, st = kda.prefill_conv(head["q"], head["k"], head["v"], head["z"], head["beta"],
                                g["A"], g["wq"], g["wk"], g["wv"], state=_states(g, True),
                                act=act, eps=EPS, S0=g["S0"])
    outs = [o]
    for t in range(T, T + extra):
        ot = kda.decode_step_conv(*(g[n][:, t].clone() for n in ("q", "k", "v", "z", "beta")),
                                  g["A"], g["wq"], g["wk"], g["wv"], st, S, act=act, eps=EPS)
        outs.append(ot[:, None])
    torch.cuda.synchronize()
    o_ref, S_ref, st_ref = _oracle_layer(inp, W, act, True)
    eo = slice_relerr(host(torch.cat(outs, dim=1)), o_ref, 2)
    es = slice_relerr(host(S), S_ref, 1)
    _say(f"[decode_conv after prefill_conv] o err {eo:.3e}  S err {es:.3e}")
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]
    _check_states(st, st_ref, W)


def test_decode_conv_k3_full_batch(kda, gpu_device):
    """K3 decode shape (B=64, H=96, bf16): two steps for every head."""
    w = WORKLOADS["k3_decode_bf16"]
    W, act = 4, "silu"
    inp = make_layer_decode_inputs(w, W, steps=2)
    _say(f"[decode_conv] {w.name} full batch, 2 steps")
    g = _dev(inp, gpu_device)
    S = torch.zeros_like(g["S"])
    st = tuple(t.clone() for t in _states(g, True))
    S_ref, st_ref = host(inp["S"]), _host_states(inp, True)
    for t in range(2):
        o = kda.decode_step_conv(g["q"][t], g["k"][t], g["v"][t], g["z"][t], g["beta"][t],
                                 g["A"], g["wq"], g["wk"], g["wv"], st, S, act=act, eps=EPS)
        torch.cuda.synchronize()
        o_ref, S_ref, st_ref = oracle.decode_step_conv(
            host(inp["q"][t]), host(inp["k"][t]), host(inp["v"][t]), host(inp["z"][t]),
            host(inp["beta"][t]), host(inp["A"]), host(inp["wq"]), host(inp["wk"]),
            host(inp["wv"]), st_ref, S_ref, act, EPS)
        eo = slice_relerr(host(o)[:, None], o_ref[:, None], 2)
        _say(f"   step {t}: o err {eo:.3e}")
        assert eo <= TOL[torch.bfloat16]
    assert slice_relerr(host(S), S_ref, 1) <= TOL[torch.bfloat16]
    _check_states(st, st_ref, W)
