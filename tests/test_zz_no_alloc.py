"""kda_prefill_varlen_noalloc: the packed prefill for callers that cannot
allocate (the ranking of the sequences lives in the library's static scratch).

Called through the C ABI twice in a row on one GPU, the second call with a
smaller input (fewer and shorter sequences), each against kda_prefill_varlen
with its caller-provided workspace: the same kernels, so the outputs must be
identical bit for bit.  More sequences than the scratch holds are refused
before anything is launched.
"""
import ctypes

import pytest
import torch

from linear_recurrent_attention_chunkwise_amd.inputs import WORKLOADS, make_varlen_inputs
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(lib, fn, g, N, T, H, chunk, o, S_T, ws=None):
    args = [1, N, T, H, 128, 128, chunk, _ptr(g["cu_seqlens"]), _ptr(g["q"]), _ptr(g["k"]),
            _ptr(g["v"]), _ptr(g["z"]), _ptr(g["beta"]), _ptr(g["A"]), _ptr(g["S0"]), _ptr(o),
            _ptr(S_T), 0, None, 0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if fn == "kda_prefill_varlen":
        args += [_ptr(ws), ws.numel() if ws is not None else 0, stream, 0]
    else:
        args += [stream, 0]
    return getattr(lib, fn)(*args)


@pytest.mark.parametrize("lengths,chunk", [([300, 17, 0, 64, 1000, 5, 129, 2048], 16),
                                           ([40, 200, 1], 64)])
def test_noalloc_matches_varlen(gpu_device, lengths, chunk, request):
    from linear_recurrent_attention_chunkwise_amd import kda as binding
    lib = binding._load()
    w = WORKLOADS["k3_prefill_bf16"].with_(H=4)
    g = to_dev(make_varlen_inputs(w, lengths), gpu_device)
    N, T, H = len(lengths), sum(lengths), w.H
    print(f"[noalloc] lengths {lengths} chunk {chunk}", flush=True)
    o1 = torch.full_like(g["v"], float("nan"))
    S1 = torch.full_like(g["S0"], float("nan"))
    assert _call(lib, "kda_prefill_varlen_noalloc", g, N, T, H, chunk, o1, S1) == 0
    o2 = torch.full_like(g["v"], float("nan"))
    S2 = torch.full_like(g["S0"], float("nan"))
    ws_bytes = int(lib.kda_prefill_varlen_workspace_size(N))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=gpu_device) if ws_bytes else None
    assert _call(lib, "kda_prefill_varlen", g, N, T, H, chunk, o2, S2, ws) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    assert torch.isfinite(S1).all()


def test_noalloc_refuses_more_sequences_than_scratch(gpu_device):
    from linear_recurrent_attention_chunkwise_amd import kda as binding
    lib = binding._load()
    N = 8193
    cu = torch.arange(N + 1, dtype=torch.int64, device=gpu_device)
    x = torch.zeros(N, 1, 128, dtype=torch.bfloat16, device=gpu_device)
    beta = torch.zeros(N, 1, dtype=torch.bfloat16, device=gpu_device)
    A = torch.zeros(1, device=gpu_device)
    o = torch.zeros_like(x)
    S_T = torch.zeros(N, 1, 128, 128, device=gpu_device)
    st = lib.kda_prefill_varlen_noalloc(1, N, N, 1, 128, 128, 16, _ptr(cu), _ptr(x), _ptr(x),
                                        _ptr(x), _ptr(x), _ptr(beta), _ptr(A), None, _ptr(o),
                                        _ptr(S_T), 0, None, 0, None, 0)
    assert st == 6   # KDA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(S_T) == 0
