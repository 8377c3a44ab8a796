"""ctypes binding over libkda.so (include/kda.h).

Argument marshalling only: shapes, dtypes, devices and contiguity are checked
here, output tensors are allocated with torch on the inputs' device, and the
call goes to the library on torch's current stream.  Every arithmetic step
runs in the library's HIP kernels.  If the library is missing, or no GPU is
visible, these functions raise; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libkda.so"

KDA_F32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KDAError(RuntimeError):
    """A libkda call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class ShortConv(ctypes.Structure):
    """kda_short_conv of include/kda.h (host struct; the taps are device memory)."""
    _fields_ = [("width", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("eps", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p)]


ACTIVATIONS = {"none": 0, "silu": 1}

_lib = None


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_prefill_workspace_size.restype = sz
    lib.kda_prefill_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32]
    pre = [ctypes.c_int, i64, i64, i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp,
           vp, vp, vp, sz, vp]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill.argtypes = pre
    lib.kda_prefill_ex.restype = ctypes.c_int
    lib.kda_prefill_ex.argtypes = pre + [i32]
    lib.kda_prefill_varlen.restype = ctypes.c_int
    lib.kda_prefill_varlen.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32, vp,
                                       vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       i32, vp, i64, vp, sz, vp, i32]
    lib.kda_prefill_varlen_noalloc.restype = ctypes.c_int
    lib.kda_prefill_varlen_noalloc.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32, vp,
                                               vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               i32, vp, i64, vp, i32]
    lib.kda_prefill_varlen_workspace_size.restype = sz
    lib.kda_prefill_varlen_workspace_size.argtypes = [i64]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [ctypes.c_int, i64, i64, i64, i64, vp, vp, vp, vp, vp,
                                    vp, vp, vp, vp]
    lib.kda_prefill_split.restype = ctypes.c_int
    lib.kda_prefill_split.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp,
                                      vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_prefill_split_workspace_size.restype = sz
    lib.kda_prefill_split_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32,
                                                     i32]
    cp = ctypes.POINTER(ShortConv)
    lib.kda_conv_norm.restype = ctypes.c_int
    lib.kda_conv_norm.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, cp, vp, vp, vp,
                                  vp, vp, vp, vp, vp, vp]
    lib.kda_conv_norm_varlen.restype = ctypes.c_int
    lib.kda_conv_norm_varlen.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, vp, cp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp]
    lib.kda_prefill_conv_workspace_size.restype = sz
    lib.kda_prefill_conv_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32]
    lib.kda_prefill_conv.restype = ctypes.c_int
    lib.kda_prefill_conv.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i32, cp,
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i32]
    lib.kda_decode_step_conv.restype = ctypes.c_int
    lib.kda_decode_step_conv.argtypes = [ctypes.c_int, i64, i64, i64, i64, cp, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp]
    lib.kda_prefill_bwd.restype = ctypes.c_int
    lib.kda_prefill_bwd.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64] + [vp] * 17 + [
        sz, vp]
    lib.kda_prefill_bwd_ex.restype = ctypes.c_int
    lib.kda_prefill_bwd_ex.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64] + [vp] * 17 + [
        sz, vp, vp]
    lib.kda_prefill_bwd_workspace_size.restype = sz
    lib.kda_prefill_bwd_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64]
    _lib = lib
    return lib


def abi_version() -> int:
    return int(_load().kda_abi_version())


def status_str(status: int) -> str:
    return _load().kda_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise KDAError(status, f"{what}: {status_str(status)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prefill_workspace_size(dtype: torch.dtype, B: int, T: int, H: int, dk: int, dv: int,
                           chunk: int) -> int:
    return int(_load().kda_prefill_workspace_size(_DTYPES[dtype], B, T, H, dk, dv, chunk))


def prefill(q, k, v, z, beta, A, S0=None, chunk: int = 16, out=None, S_T=None,
            dv_per_block: int = 0, segments: int = 1, workspace=None):
    """Chunkwise KDA prefill on the GPU.

    q, k, z [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H] (fp32 or bf16, all one
    dtype); A [H] fp32; S0 [B,H,dk,dv] fp32 or None.  Returns (o, S_T) with
    o [B,T,H,dv] in the input dtype and S_T [B,H,dk,dv] fp32.  ``out`` and
    ``S_T`` may be given preallocated (``S_T`` may be ``S0`` itself).
    ``segments`` > 1 splits every sequence into that many pieces run in
    parallel and combined through their state maps (kda_prefill_split; bf16,
    d = 128, chunk 16 or 64); ``workspace`` may then be a preallocated uint8 cuda
    tensor of ``prefill_split_workspace_size`` bytes."""
    lib = _load()
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("KDA prefill runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _require(q, "q", (B, T, H, dk), dt, dev)
    _require(k, "k", (B, T, H, dk), dt, dev)
    _require(z, "z", (B, T, H, dk), dt, dev)
    _require(v, "v", (B, T, H, dv), dt, dev)
    _require(beta, "beta", (B, T, H), dt, dev)
    _require(A, "A", (H,), torch.float32, dev)
    if S0 is not None:
        _require(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _require(out, "out", (B, T, H, dv), dt, dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _require(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    if segments > 1:
        ws_bytes = prefill_split_workspace_size(dt, B, T, H, dk, dv, chunk, segments)
        if workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        elif workspace.numel() < ws_bytes or workspace.device != dev:
            raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
        st = lib.kda_prefill_split(_DTYPES[dt], B, T, H, dk, dv, int(chunk), int(segments),
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                   _ptr(S0), _ptr(out), _ptr(S_T), _ptr(workspace),
                                   workspace.numel() if workspace is not None else 0,
                                   _stream_handle(dev))
        _check(st, "kda_prefill_split")
        return out, S_T
    ws_bytes = int(lib.kda_prefill_workspace_size(_DTYPES[dt], B, T, H, dk, dv, int(chunk)))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    args = [_DTYPES[dt], B, T, H, dk, dv, int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(z),
            _ptr(beta), _ptr(A), _ptr(S0), _ptr(out), _ptr(S_T), _ptr(ws), ws_bytes,
            _stream_handle(dev)]
    if dv_per_block:   # an explicit column split: the _ex entry point
        _check(lib.kda_prefill_ex(*args, int(dv_per_block)), "kda_prefill_ex")
    else:
        _check(lib.kda_prefill(*args), "kda_prefill")
    return out, S_T


def prefill_split_workspace_size(dtype: torch.dtype, B: int, T: int, H: int, dk: int, dv: int,
                                 chunk: int, segments: int) -> int:
    return int(_load().kda_prefill_split_workspace_size(_DTYPES[dtype], B, T, H, dk, dv,
                                                        int(chunk), int(segments)))


def checkpoint_rows(seq_lens, ckpt_every: int):
    """First checkpoint row of each sequence and the total row count, for the
    layout of ``prefill_varlen``: floor(L_i / ckpt_every) rows per sequence,
    in sequence order."""
    rows, r0 = [], 0
    for L in seq_lens:
        rows.append(r0)
        r0 += int(L) // ckpt_every if ckpt_every > 0 else 0
    return rows, r0


def prefill_varlen(q, k, v, z, beta, A, cu_seqlens, S0=None, chunk: int = 16,
                   ckpt_every: int = 0, out=None, S_T=None, ckpt=None,
                   dv_per_block: int = 0, seq_lens=None, no_alloc: bool = False):
    """KDA prefill over N sequences packed along one token axis.

    q, k, z [T,H,dk]; v [T,H,dv]; beta [T,H] (one dtype, fp32 or bf16);
    A [H] fp32; cu_seqlens int64 [N+1] (sequence i is tokens
    cu_seqlens[i]:cu_seqlens[i+1]); S0 [N,H,dk,dv] fp32 or None.
    ckpt_every > 0 (a multiple of ``chunk``) also returns the state after every
    ckpt_every tokens of each sequence: ckpt [R,H,dk,dv] fp32, rows in sequence
    order (see ``checkpoint_rows``).  Returns (o, S_T, ckpt-or-None).

    ``cu_seqlens`` may be a CPU or GPU tensor; the library reads a GPU copy,
    and host values size the checkpoint buffer.  Passing ``seq_lens`` (the
    host list of lengths) together with a GPU ``cu_seqlens`` avoids every
    host-device copy in this call.

    ``no_alloc=True`` calls kda_prefill_varlen_noalloc, which ranks the
    sequences in the library's static scratch instead of a workspace (at most
    8192 sequences); with ``out``, ``S_T`` (and ``ckpt``) given and a GPU
    ``cu_seqlens`` with ``seq_lens``, the call then allocates nothing."""
    lib = _load()
    if q.dim() != 3:
        raise ValueError("q must be [T,H,dk] (packed sequences)")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("KDA prefill runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    if not isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = torch.tensor(list(cu_seqlens), dtype=torch.int64)
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor [N+1]")
    if seq_lens is not None and cu_seqlens.device == dev:
        lens = [int(L) for L in seq_lens]
        if len(lens) != cu_seqlens.numel() - 1 or any(L < 0 for L in lens) or sum(lens) != T:
            raise ValueError("seq_lens must hold N non-negative lengths summing to T")
        cu_dev = cu_seqlens.contiguous()
    else:
        cu_host = cu_seqlens.cpu()
        lens = (cu_host[1:] - cu_host[:-1]).tolist()
        if int(cu_host[0]) != 0 or any(L < 0 for L in lens) or int(cu_host[-1]) != T:
            raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
        cu_dev = cu_seqlens.to(dev).contiguous()
    N = len(lens)
    _require(q, "q", (T, H, dk), dt, dev)
    _require(k, "k", (T, H, dk), dt, dev)
    _require(z, "z", (T, H, dk), dt, dev)
    _require(v, "v", (T, H, dv), dt, dev)
    _require(beta, "beta", (T, H), dt, dev)
    _require(A, "A", (H,), torch.float32, dev)
    if S0 is not None:
        _require(S0, "S0", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    _require(out, "out", (T, H, dv), dt, dev)
    if S_T is None:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    _require(S_T, "S_T", (N, H, dk, dv), torch.float32, dev)
    n_ckpt = 0
    if ckpt_every > 0:
        _, n_ckpt = checkpoint_rows(lens, int(ckpt_every))
        if ckpt is None:
            ckpt = torch.empty((n_ckpt, H, dk, dv), dtype=torch.float32, device=dev)
        _require(ckpt, "ckpt", (n_ckpt, H, dk, dv), torch.float32, dev)
    else:
        ckpt = None
    if no_alloc:
        st = lib.kda_prefill_varlen_noalloc(_DTYPES[dt], N, T, H, dk, dv, int(chunk), _ptr(cu_dev),
                                            _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta),
                                            _ptr(A), _ptr(S0), _ptr(out), _ptr(S_T),
                                            int(ckpt_every), _ptr(ckpt), n_ckpt,
                                            _stream_handle(dev), int(dv_per_block))
        _check(st, "kda_prefill_varlen_noalloc")
        return out, S_T, ckpt
    ws_bytes = int(lib.kda_prefill_varlen_workspace_size(N))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    st = lib.kda_prefill_varlen(_DTYPES[dt], N, T, H, dk, dv, int(chunk), _ptr(cu_dev),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A),
                                _ptr(S0), _ptr(out), _ptr(S_T), int(ckpt_every), _ptr(ckpt),
                                n_ckpt, _ptr(ws), ws_bytes, _stream_handle(dev),
                                int(dv_per_block))
    _check(st, "kda_prefill_varlen")
    return out, S_T, ckpt


def decode_step(q, k, v, z, beta, A, S, out=None):
    """One fused KDA decode step on the GPU; S [B,H,dk,dv] fp32 is updated in
    place.  q, k, z [B,H,dk]; v [B,H,dv]; beta [B,H]; A [H] fp32.  Returns o
    [B,H,dv] in the input dtype."""
    lib = _load()
    if q.dim() != 3:
        raise ValueError("q must be [B,H,dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("KDA decode runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _require(q, "q", (B, H, dk), dt, dev)
    _require(k, "k", (B, H, dk), dt, dev)
    _require(z, "z", (B, H, dk), dt, dev)
    _require(v, "v", (B, H, dv), dt, dev)
    _require(beta, "beta", (B, H), dt, dev)
    _require(A, "A", (H,), torch.float32, dev)
    _require(S, "S", (B, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, H, dv), dtype=dt, device=dev)
    _require(out, "out", (B, H, dv), dt, dev)
    st = lib.kda_decode_step(_DTYPES[dt], B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(z),
                             _ptr(beta), _ptr(A), _ptr(S), _ptr(out), _stream_handle(dev))
    _check(st, "kda_decode_step")
    return out


# ------------------------------------------------------------- prologue ----

def _short_conv(wq, wk, wv, act, eps, H, dk, dv, dev):
    if not isinstance(wq, torch.Tensor) or wq.dim() != 3:
        raise ValueError("wq must be [H,dk,W]")
    W = wq.shape[-1]
    _require(wq, "wq", (H, dk, W), torch.float32, dev)
    _require(wk, "wk", (H, dk, W), torch.float32, dev)
    _require(wv, "wv", (H, dv, W), torch.float32, dev)
    if act not in ACTIVATIONS:
        raise ValueError(f"act must be one of {sorted(ACTIVATIONS)}")
    cs = ShortConv(int(W), ACTIVATIONS[act], float(eps), 0, wq.data_ptr(), wk.data_ptr(),
                   wv.data_ptr())
    return cs, int(W)


def _states(states, name, B, W, H, dk, dv, dt, dev):
    """(sq, sk, sv) tensors [B,W-1,H,d] -> host array of 3 device pointers."""
    if states is None:
        return None
    sq, sk, sv = states
    _require(sq, f"{name}[0]", (B, W - 1, H, dk), dt, dev)
    _require(sk, f"{name}[1]", (B, W - 1, H, dk), dt, dev)
    _require(sv, f"{name}[2]", (B, W - 1, H, dv), dt, dev)
    return (ctypes.c_void_p * 3)(sq.data_ptr(), sk.data_ptr(), sv.data_ptr())


def _new_states(B, W, H, dk, dv, dt, dev):
    return tuple(torch.empty((B, W - 1, H, d), dtype=dt, device=dev) for d in (dk, dk, dv))


def _seg_shapes(q, v, what):
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError(f"{what} runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    return B, T, H, dk, v.shape[-1], dev, dt


def conv_norm(q, k, v, wq, wk, wv, state=None, act: str = "none", eps: float = 1e-6,
              out=None, state_out=True):
    """The layer prologue on the GPU: causal depthwise convolutions of raw q, k, v
    (taps wq, wk [H,dk,W], wv [H,dv,W] fp32), optional SiLU, then q, k
    L2-normalized.  ``state`` is None (fresh sequences) or (sq, sk, sv), each
    [B,W-1,H,d] in the input dtype.  Returns (q_hat, k_hat, v_conv, new_state);
    new_state is a fresh tuple when ``state_out`` is True, the given tuple when
    one is passed, None when False."""
    lib = _load()
    B, T, H, dk, dv, dev, dt = _seg_shapes(q, v, "the KDA prologue")
    _require(q, "q", (B, T, H, dk), dt, dev)
    _require(k, "k", (B, T, H, dk), dt, dev)
    _require(v, "v", (B, T, H, dv), dt, dev)
    cs, W = _short_conv(wq, wk, wv, act, eps, H, dk, dv, dev)
    sin = _states(state, "state", B, W, H, dk, dv, dt, dev)
    if state_out is True:
        state_out = _new_states(B, W, H, dk, dv, dt, dev)
    elif state_out is False:
        state_out = None
    sout = _states(state_out, "state_out", B, W, H, dk, dv, dt, dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for t, ref, name in zip(out, (q, k, v), ("q_out", "k_out", "v_out")):
        _require(t, name, tuple(ref.shape), dt, dev)
    st = lib.kda_conv_norm(_DTYPES[dt], B, T, H, dk, dv, ctypes.byref(cs), _ptr(q), _ptr(k),
                           _ptr(v), sin, sout, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
                           _stream_handle(dev))
    _check(st, "kda_conv_norm")
    return out[0], out[1], out[2], state_out


def conv_norm_varlen(q, k, v, wq, wk, wv, cu_seqlens, state=None, act: str = "none",
                     eps: float = 1e-6, out=None, state_out=True):
    """The prologue over N packed sequences: q, k [T,H,dk], v [T,H,dv];
    cu_seqlens int64 [N+1] (a cuda tensor, or host values copied over);
    ``state`` None or (sq, sk, sv) each [N,W-1,H,d].  Returns (q_hat, k_hat,
    v_conv, new_state) as ``conv_norm`` does."""
    lib = _load()
    if q.dim() != 3:
        raise ValueError("q must be [T,H,dk] (packed sequences)")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("the KDA prologue runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    if not isinstance(cu_seqlens, torch.Tensor):
        cu_seqlens = torch.tensor(list(cu_seqlens), dtype=torch.int64)
    if cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int64 tensor [N+1]")
    cu_dev = cu_seqlens.to(dev).contiguous()
    N = cu_dev.numel() - 1
    _require(q, "q", (T, H, dk), dt, dev)
    _require(k, "k", (T, H, dk), dt, dev)
    _require(v, "v", (T, H, dv), dt, dev)
    cs, W = _short_conv(wq, wk, wv, act, eps, H, dk, dv, dev)
    sin = _states(state, "state", N, W, H, dk, dv, dt, dev)
    if state_out is True:
        state_out = _new_states(N, W, H, dk, dv, dt, dev)
    elif state_out is False:
        state_out = None
    sout = _states(state_out, "state_out", N, W, H, dk, dv, dt, dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for t, ref, name in zip(out, (q, k, v), ("q_out", "k_out", "v_out")):
        _require(t, name, tuple(ref.shape), dt, dev)
    st = lib.kda_conv_norm_varlen(_DTYPES[dt], N, T, H, dk, dv, _ptr(cu_dev), ctypes.byref(cs),
                                  _ptr(q), _ptr(k), _ptr(v), sin, sout, _ptr(out[0]),
                                  _ptr(out[1]), _ptr(out[2]), _stream_handle(dev))
    _check(st, "kda_conv_norm_varlen")
    return out[0], out[1], out[2], state_out


def prefill_conv_workspace_size(dtype: torch.dtype, B: int, T: int, H: int, dk: int, dv: int,
                                chunk: int) -> int:
    return int(_load().kda_prefill_conv_workspace_size(_DTYPES[dtype], B, T, H, dk, dv, chunk))


def prefill_conv(q, k, v, z, beta, A, wq, wk, wv, state=None, act: str = "none",
                 eps: float = 1e-6, S0=None, chunk: int = 16, out=None, S_T=None,
                 state_out=True, workspace=None, dv_per_block: int = 0):
    """Prologue + chunkwise prefill of raw q, k, v (see ``conv_norm`` and
    ``prefill``).  Returns (o, S_T, new_state).  ``workspace`` may be a
    preallocated uint8 cuda tensor of at least ``prefill_conv_workspace_size``
    bytes."""
    lib = _load()
    B, T, H, dk, dv, dev, dt = _seg_shapes(q, v, "KDA prefill")
    _require(q, "q", (B, T, H, dk), dt, dev)
    _require(k, "k", (B, T, H, dk), dt, dev)
    _require(z, "z", (B, T, H, dk), dt, dev)
    _require(v, "v", (B, T, H, dv), dt, dev)
    _require(beta, "beta", (B, T, H), dt, dev)
    _require(A, "A", (H,), torch.float32, dev)
    if S0 is not None:
        _require(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    cs, W = _short_conv(wq, wk, wv, act, eps, H, dk, dv, dev)
    sin = _states(state, "state", B, W, H, dk, dv, dt, dev)
    if state_out is True:
        state_out = _new_states(B, W, H, dk, dv, dt, dev)
    elif state_out is False:
        state_out = None
    sout = _states(state_out, "state_out", B, W, H, dk, dv, dt, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    _require(out, "out", (B, T, H, dv), dt, dev)
    if S_T is None:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    _require(S_T, "S_T", (B, H, dk, dv), torch.float32, dev)
    ws_bytes = prefill_conv_workspace_size(dt, B, T, H, dk, dv, chunk)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    elif workspace.numel() < ws_bytes or workspace.device != dev:
        raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    st = lib.kda_prefill_conv(_DTYPES[dt], B, T, H, dk, dv, int(chunk), ctypes.byref(cs),
                              _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A), sin, sout,
                              _ptr(S0), _ptr(out), _ptr(S_T), _ptr(workspace),
                              workspace.numel() if workspace is not None else 0,
                              _stream_handle(dev), int(dv_per_block))
    _check(st, "kda_prefill_conv")
    return out, S_T, state_out


def decode_step_conv(q, k, v, z, beta, A, wq, wk, wv, state, S, act: str = "none",
                     eps: float = 1e-6, out=None):
    """One decode step with the prologue fused in.  q, k, z [B,H,dk], v [B,H,dv]
    raw; ``state`` = (sq, sk, sv) [B,W-1,H,d] and S [B,H,dk,dv] fp32 are
    updated in place.  Returns o [B,H,dv]."""
    lib = _load()
    if q.dim() != 3:
        raise ValueError("q must be [B,H,dk]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("KDA decode runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _require(q, "q", (B, H, dk), dt, dev)
    _require(k, "k", (B, H, dk), dt, dev)
    _require(z, "z", (B, H, dk), dt, dev)
    _require(v, "v", (B, H, dv), dt, dev)
    _require(beta, "beta", (B, H), dt, dev)
    _require(A, "A", (H,), torch.float32, dev)
    _require(S, "S", (B, H, dk, dv), torch.float32, dev)
    cs, W = _short_conv(wq, wk, wv, act, eps, H, dk, dv, dev)
    sarr = _states(state, "state", B, W, H, dk, dv, dt, dev) if W > 1 else None
    if out is None:
        out = torch.empty((B, H, dv), dtype=dt, device=dev)
    _require(out, "out", (B, H, dv), dt, dev)
    st = lib.kda_decode_step_conv(_DTYPES[dt], B, H, dk, dv, ctypes.byref(cs), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A), sarr,
                                  _ptr(S), _ptr(out), _stream_handle(dev))
    _check(st, "kda_decode_step_conv")
    return out


def prefill_bwd_workspace_size(dtype: torch.dtype, B: int, T: int, H: int, dk: int,
                               dv: int) -> int:
    return int(_load().kda_prefill_bwd_workspace_size(_DTYPES[dtype], B, T, H, dk, dv))


_side_streams = {}


def _side_stream(dev):
    """One torch stream per device (default priority) for the backward's
    overlapped prep; owned here, on the caller's side of the C ABI."""
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if idx not in _side_streams:
        _side_streams[idx] = torch.cuda.Stream(device=idx)
    return _side_streams[idx]


def prefill_bwd(q, k, v, z, beta, A, S0, dO, dS_T=None, workspace=None, side_stream="auto"):
    """Gradients of a loss through the prefill (kda_prefill_bwd_ex).

    Inputs as ``prefill`` (S0 may be None), dO [B,T,H,dv] in the input dtype
    (dL/do) and dS_T [B,H,dk,dv] fp32 or None (dL/dS_T).  Returns a dict of
    fp32 tensors: dq, dk, dz [B,T,H,dk]; dv [B,T,H,dv]; dbeta [B,T,H];
    dA [H]; dS0 [B,H,dk,dv].  ``workspace`` may be a preallocated uint8 cuda
    tensor of ``prefill_bwd_workspace_size`` bytes.  ``side_stream``: a
    torch.cuda.Stream on which the library may run its prep kernel beside the
    forward rerun, ``"auto"`` (a stream kept by this module, one per device)
    or None (everything on the current stream; the same results)."""
    lib = _load()
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    if dev.type != "cuda":
        raise ValueError("KDA backward runs on the GPU; inputs must be cuda tensors")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _require(q, "q", (B, T, H, dk), dt, dev)
    _require(k, "k", (B, T, H, dk), dt, dev)
    _require(z, "z", (B, T, H, dk), dt, dev)
    _require(v, "v", (B, T, H, dv), dt, dev)
    _require(beta, "beta", (B, T, H), dt, dev)
    _require(A, "A", (H,), torch.float32, dev)
    _require(dO, "dO", (B, T, H, dv), dt, dev)
    if S0 is not None:
        _require(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    if dS_T is not None:
        _require(dS_T, "dS_T", (B, H, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
         "dv": torch.empty((B, T, H, dv), **f32), "dz": torch.empty((B, T, H, dk), **f32),
         "dbeta": torch.empty((B, T, H), **f32), "dA": torch.empty((H,), **f32),
         "dS0": torch.empty((B, H, dk, dv), **f32)}
    ws_bytes = prefill_bwd_workspace_size(dt, B, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    elif workspace.numel() < ws_bytes or workspace.device != dev:
        raise ValueError(f"workspace must hold {ws_bytes} bytes on {dev}")
    if isinstance(side_stream, str):
        if side_stream != "auto":
            raise ValueError("side_stream must be a torch.cuda.Stream, 'auto' or None")
        side_stream = _side_stream(dev)
    side = ctypes.c_void_p(side_stream.cuda_stream) if side_stream is not None else None
    st = lib.kda_prefill_bwd_ex(_DTYPES[dt], B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(z), _ptr(beta), _ptr(A), _ptr(S0), _ptr(dO), _ptr(dS_T),
                                _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dz"]),
                                _ptr(g["dbeta"]), _ptr(g["dA"]), _ptr(g["dS0"]), _ptr(workspace),
                                workspace.numel() if workspace is not None else 0,
                                _stream_handle(dev), side)
    _check(st, "kda_prefill_bwd_ex")
    return g
