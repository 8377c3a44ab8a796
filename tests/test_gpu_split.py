"""GPU parity of the sequence-split prefill (kda_prefill_split): each sequence
cut into segments that run in parallel, their start states recovered through
the segments' affine state maps (S_end = M S_start + N).

Against the fp64 oracle at the tolerances of the plain prefill (2e-2 for bf16
inputs, normwise per (b, h) slice), over ragged lengths, segment counts that
leave trailing segments empty, a long-memory variant (decays near 1, so the
maps M carry the state across many segments) and in-place state carry, at
both chunk lengths (16: the role-split kernel, M and N on one pass; 64: the
general kernel, M and N as runs of their own).  The million-token head share
is tested in test_gpu_million.py.
"""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_chunkwise_amd.inputs import WORKLOADS, make_prefill_inputs
from tests.gpu_helpers import TOL, gpu_prefill, host, oracle_prefill, slice_relerr, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    import linear_recurrent_attention_chunkwise_amd as m
    assert m.abi_version() == 8
    return m


def _say(*a):
    print(*a, flush=True)


def _split(kda, g, P, chunk=16, **kw):
    o, S_T = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], g["S0"], chunk=chunk,
                         segments=P, **kw)
    torch.cuda.synchronize()
    return o, S_T


@pytest.mark.parametrize("chunk", [16, 64])
@pytest.mark.parametrize("P", [2, 3, 7])
def test_split_matches_oracle(kda, gpu_device, P, chunk):
    w = WORKLOADS["k3_prefill_bf16"].with_(B=2, H=2, s0_std=0.5)
    for T in (1, 17, 100, 333, 1000):
        inp = make_prefill_inputs(w, T=T)
        _say(f"[split] B=2 H=2 T={T} segments={P} chunk={chunk}")
        o, S_T = _split(kda, to_dev(inp, gpu_device), P, chunk)
        o_ref, S_ref = oracle_prefill(inp)
        eo, es = slice_relerr(host(o), o_ref, 2), slice_relerr(host(S_T), S_ref, 1)
        _say(f"   o err {eo:.3e}  S_T err {es:.3e}")
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


@pytest.mark.parametrize("chunk", [16, 64])
def test_split_long_memory(kda, gpu_device, chunk):
    """z ~ N(-6, 1): alpha in 0.6..1, so a segment's state map M is far from 0
    and the scan really carries the state across segments."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=1, H=3, z_mean=-6.0, s0_std=0.5)
    inp = make_prefill_inputs(w, T=2048)
    for P in (4, 8, 16):
        _say(f"[split] long memory T=2048 segments={P} chunk={chunk}")
        o, S_T = _split(kda, to_dev(inp, gpu_device), P, chunk)
        o_ref, S_ref = oracle_prefill(inp)
        eo, es = slice_relerr(host(o), o_ref, 2), slice_relerr(host(S_T), S_ref, 1)
        _say(f"   o err {eo:.3e}  S_T err {es:.3e}")
        assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


@pytest.mark.parametrize("chunk", [16, 64])
def test_split_empty_segments_and_edges(kda, gpu_device, chunk):
    """T = 0 returns S0; T smaller than the segment count leaves trailing
    segments empty; S_T may be S0 itself."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=2, H=2, s0_std=0.5)
    g = to_dev(make_prefill_inputs(w, T=0), gpu_device)
    o, S_T = _split(kda, g, 4, chunk)
    assert torch.equal(S_T, g["S0"])
    # segments of one chunk: 2 used, 14 empty
    inp = make_prefill_inputs(w, T=chunk + 4)
    g = to_dev(inp, gpu_device)
    o, S_T = _split(kda, g, 16, chunk)
    o_ref, S_ref = oracle_prefill(inp)
    assert slice_relerr(host(o), o_ref, 2) <= 2e-2 and slice_relerr(host(S_T), S_ref, 1) <= 2e-2
    # in place
    S = g["S0"].clone()
    o2, S2 = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], S, chunk=chunk,
                         segments=16, S_T=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr() and torch.equal(S2, S_T) and torch.equal(o2, o)


@pytest.mark.parametrize("chunk", [16, 64])
def test_split_first_segment_is_exact(kda, gpu_device, chunk):
    """The first segment starts from S0 itself, so its outputs are the unsplit
    run's bits; later segments differ only by rounding."""
    w = WORKLOADS["k3_prefill_bf16"].with_(B=1, H=4, s0_std=0.02)
    g = to_dev(make_prefill_inputs(w, T=4096), gpu_device)
    o, S_T = _split(kda, g, 4, chunk)
    o0, S0_ = gpu_prefill(kda, g, chunk, dv_per_block=64 if chunk == 16 else 128)
    assert torch.equal(o[:, :1024], o0[:, :1024])
    eo = slice_relerr(host(o), host(o0), 2)
    es = slice_relerr(host(S_T), host(S0_), 1)
    _say(f"[split] 4 segments vs unsplit: o {eo:.3e}  S_T {es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2
