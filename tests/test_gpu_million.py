"""GPU parity on the million-token head share: B1 H16 T2^20 d128 bf16, one
GPU's share of a context of 1,048,576 tokens (the context length stated for
K3 in "Kimi K3 Open Weights: What Is Actually New", section "Start with the
released configuration").

Both chunk lengths and the sequence split at each (8 segments at chunk 16,
9 and 17 at chunk 64) are compared with the
fp64 oracle over the FULL length on two heads (the oracle runs segment by
segment with the state carried across, which the split invariant pins on the
oracle itself), normwise per head at the bf16 tolerance 2e-2.  On top of
that, each unsplit run is checked bit for bit against two half-length runs
chained through the state (outputs are causal, and 2^19 is a multiple of
both chunk lengths, so the halves must reproduce the same bits).
"""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_chunkwise_amd.inputs import WORKLOADS, make_prefill_inputs
from tests.gpu_helpers import diag, gpu_prefill, host, oracle_prefill_chained, slice_relerr

pytestmark = pytest.mark.gpu

HEADS = [3, 12]


@pytest.fixture(scope="module")
def kda():
    import linear_recurrent_attention_chunkwise_amd as m
    assert m.abi_version() == 8
    return m


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def million(gpu_device):
    w = WORKLOADS["million_prefill_bf16"]
    _say(f"[million] {w.name}: drawing inputs on the GPU")
    inp = make_prefill_inputs(w, device=gpu_device)
    _say(f"[million] oracle over all {w.T} tokens of heads {HEADS} (chained segments)")
    o_ref, S_ref = oracle_prefill_chained(inp, HEADS)
    _say("[million] oracle done")
    return w, inp, o_ref, S_ref


def _against_oracle(o, S_T, o_ref, S_ref, what):
    idx = torch.as_tensor(HEADS, device=o.device)
    o_h = host(torch.index_select(o, 2, idx))
    S_h = host(torch.index_select(S_T, 1, idx))
    eo = slice_relerr(o_h, o_ref, 2)
    es = slice_relerr(S_h, S_ref, 1)
    _say(f"   {what}: o err {eo:.3e}  S_T err {es:.3e}  ({diag(o_h, o_ref)})")
    assert eo <= 2e-2 and es <= 2e-2, what
    assert torch.isfinite(S_T).all()


@pytest.mark.parametrize("chunk", [16, 64])
def test_million_token_prefill(kda, gpu_device, million, chunk):
    w, inp, o_ref, S_ref = million
    _say(f"[million] unsplit, chunk {chunk}")
    o, S_T = gpu_prefill(kda, inp, chunk)
    _against_oracle(o, S_T, o_ref, S_ref, f"chunk {chunk} vs oracle")
    half = w.T // 2
    first = {k: (v[:, :half].clone() if v is not None and v.dim() >= 3 else v)
             for k, v in inp.items()}
    o1, S1 = gpu_prefill(kda, first, chunk)
    assert torch.equal(o1, o[:, :half])
    del first, o1
    second = {k: (v[:, half:].clone() if v is not None and v.dim() >= 3 else v)
              for k, v in inp.items()}
    second["S0"] = S1
    o2, S2 = gpu_prefill(kda, second, chunk)
    assert torch.equal(o2, o[:, half:]) and torch.equal(S2, S_T)
    _say("   halves chained through S reproduce the bits")


def _head_relerr(x, ref):
    """max over heads of max|x - ref| / max|ref| over (b, t, d), on the GPU."""
    worst = 0.0
    for h in range(ref.shape[2]):
        a = x[:, :, h].float()
        b = ref[:, :, h].float()
        worst = max(worst, ((a - b).abs().max() / b.abs().max()).item())
    return worst


@pytest.mark.parametrize("chunk,P", [(16, 4), (16, 8), (16, 9), (64, 9), (64, 17)])
def test_million_token_split(kda, gpu_device, million, chunk, P):
    """Split into P segments (chunk 16: 256 workgroups instead of 32; chunk
    64: 240 + 128 workgroups at 9 segments and 496 + 256 at 17, instead of
    16): against
    the oracle on the two full-length heads, against the unsplit run on all 16
    heads, and the first segment bit for bit (it starts from S0 itself)."""
    w, inp, o_ref, S_ref = million
    _say(f"[million] split into {P} segments, chunk {chunk}")
    o, S_T = kda.prefill(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta"], inp["A"],
                         inp["S0"], chunk=chunk, segments=P)
    torch.cuda.synchronize()
    _against_oracle(o, S_T, o_ref, S_ref, f"{P} segments vs oracle")
    o0, S0_ = gpu_prefill(kda, inp, chunk, dv_per_block=64 if chunk == 16 else 128)
    L = -(-w.T // P)
    L = -(-L // chunk) * chunk   # segment length: a whole number of chunks
    assert torch.equal(o[:, :L], o0[:, :L])
    eo = _head_relerr(o, o0)
    es = slice_relerr(host(S_T), host(S0_), 1)
    _say(f"   {P} segments vs unsplit, all heads: o {eo:.3e}  S_T {es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2
