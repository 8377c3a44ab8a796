"""Seeded synthetic KDA workloads.

This module only draws inputs; it contains none of the KDA arithmetic (no
gate, no recurrence).  Both the GPU tests and the oracle-side tests take their
inputs from here, so it must stay free of anything either side computes.

Recipe (per workload, one torch generator seeded with the workload's seed,
fp32 draws in this order):
  q, k ~ N(0,1) [.., dk], then L2-normalised over dk per (b, t, h);
  v ~ N(0,1) [.., dv];
  beta = logistic(N(0,1)) per (b, t, h);
  z ~ N(z_mean, 1) per key channel;
  A ~ U(-1, 1) per head (fp32);
  S0 ~ N(0, s0_std^2) per state entry (fp32) when s0_std is set, else zeros.
q, k, v, z, beta are then rounded to the run dtype (round-to-nearest-even for
bf16); A and S0 stay fp32.  Decode workloads draw every step up front with a
leading [steps] axis and start from a zero state.

Cotangents for the backward come from a second generator seeded with the
workload's seed + 1000: dO ~ N(0, 1) [B, T, H, dv] rounded to the run dtype,
then dL/dS_T ~ N(0, 1) [B, H, dk, dv] (fp32), i.e. the gradient of a loss
<dO, o> + <dS_T, S_T> with unit-scale random weights.

Layer inputs for the prologue (short convolutions + q/k normalization) follow
the same recipe without the L2 normalization of q and k (the prologue
normalizes), then draw, from the same generator: taps wq, wk, wv ~ N(0, 1/W)
[H, d, W] (fp32), then convolution states ~ N(0, 1) [B, W-1, H, d] rounded to
the run dtype (a sequence that continues earlier tokens).  The pages give no
tap distribution; N(0, 1/W) keeps the convolution's output at unit scale.

The workload shapes follow the Kimi K3 KDA context quoted on the pages
(96 heads, 128-dim heads, a 1,048,576-token context limit); the head count and
head size of the KDA layers are not stated there and are assumed equal to the
attention head shape.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch

__all__ = ["Workload", "WORKLOADS", "make_prefill_inputs", "make_decode_inputs", "make_varlen_inputs",
           "make_layer_inputs", "make_layer_decode_inputs", "make_cotangents", "torch_dtype"]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    H: int
    dk: int
    dv: int
    dtype: str           # "f32" or "bf16"
    seed: int
    T: int = 0           # prefill tokens
    chunk: int = 16      # prefill chunk length
    steps: int = 0       # decode steps
    z_mean: float = 0.0
    s0_std: float | None = None

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_prefill_f32", "prefill", B=1, H=2, T=64, dk=16, dv=16,
                 chunk=16, dtype="f32", seed=0),
        Workload("k3_prefill_bf16", "prefill", B=1, H=96, T=4096, dk=128, dv=128,
                 chunk=16, dtype="bf16", seed=1, s0_std=0.02),
        Workload("k3_decode_bf16", "decode", B=64, H=96, dk=128, dv=128, steps=256,
                 dtype="bf16", seed=2),
        Workload("long_prefill_bf16", "prefill", B=1, H=96, T=65536, dk=128, dv=128,
                 chunk=64, dtype="bf16", seed=3, z_mean=2.0),
        Workload("million_prefill_bf16", "prefill", B=1, H=16, T=1 << 20, dk=128,
                 dv=128, chunk=64, dtype="bf16", seed=4),
    ]
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_prefill_inputs(w: Workload, device="cpu", T: int | None = None):
    """Inputs of a prefill workload as a dict of tensors on ``device``.

    ``T`` overrides the workload's token count (same recipe and seed)."""
    T = w.T if T is None else int(T)
    g = _gen(w.seed, device)
    dt = torch_dtype(w.dtype)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    q = torch.randn(w.B, T, w.H, w.dk, **f32)
    k = torch.randn(w.B, T, w.H, w.dk, **f32)
    v = torch.randn(w.B, T, w.H, w.dv, **f32)
    beta_logit = torch.randn(w.B, T, w.H, **f32)
    z = torch.randn(w.B, T, w.H, w.dk, **f32)
    if w.z_mean:
        z.add_(w.z_mean)
    A = torch.rand(w.H, **f32).mul_(2.0).sub_(1.0)
    S0 = None
    if w.s0_std is not None:
        S0 = torch.randn(w.B, w.H, w.dk, w.dv, **f32).mul_(w.s0_std)
    q = _unit(q).to(dt)
    k = _unit(k).to(dt)
    return dict(q=q, k=k, v=v.to(dt), z=z.to(dt),
                beta=torch.sigmoid(beta_logit).to(dt), A=A, S0=S0)


def make_decode_inputs(w: Workload, device="cpu", steps: int | None = None):
    """Per-step decode inputs with a leading [steps] axis, plus A and a zero S."""
    steps = w.steps if steps is None else int(steps)
    g = _gen(w.seed, device)
    dt = torch_dtype(w.dtype)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    q = torch.randn(steps, w.B, w.H, w.dk, **f32)
    k = torch.randn(steps, w.B, w.H, w.dk, **f32)
    v = torch.randn(steps, w.B, w.H, w.dv, **f32)
    beta_logit = torch.randn(steps, w.B, w.H, **f32)
    z = torch.randn(steps, w.B, w.H, w.dk, **f32)
    if w.z_mean:
        z.add_(w.z_mean)
    A = torch.rand(w.H, **f32).mul_(2.0).sub_(1.0)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=device)
    return dict(q=_unit(q).to(dt), k=_unit(k).to(dt), v=v.to(dt), z=z.to(dt),
                beta=torch.sigmoid(beta_logit).to(dt), A=A, S=S)


def make_varlen_inputs(w: Workload, lengths, device="cpu"):
    """Packed inputs for sequences of the given lengths, drawn as one workload.

    Token tensors come from the prefill recipe with B=1 and T=sum(lengths),
    laid out [T, H, d] (``beta`` [T, H]); then one initial state per sequence
    ([N, H, dk, dv], N(0, s0_std^2) when s0_std is set, else zeros) from the
    same generator stream.  ``cu_seqlens`` is the int64 [N+1] prefix sum."""
    lengths = [int(L) for L in lengths]
    T = sum(lengths)
    g = _gen(w.seed, device)
    dt = torch_dtype(w.dtype)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    q = torch.randn(T, w.H, w.dk, **f32)
    k = torch.randn(T, w.H, w.dk, **f32)
    v = torch.randn(T, w.H, w.dv, **f32)
    beta_logit = torch.randn(T, w.H, **f32)
    z = torch.randn(T, w.H, w.dk, **f32)
    if w.z_mean:
        z.add_(w.z_mean)
    A = torch.rand(w.H, **f32).mul_(2.0).sub_(1.0)
    N = len(lengths)
    if w.s0_std is not None:
        S0 = torch.randn(N, w.H, w.dk, w.dv, **f32).mul_(w.s0_std)
    else:
        S0 = torch.zeros(N, w.H, w.dk, w.dv, dtype=torch.float32, device=device)
    cu = torch.zeros(N + 1, dtype=torch.int64)
    if N:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0)
    return dict(q=_unit(q).to(dt), k=_unit(k).to(dt), v=v.to(dt), z=z.to(dt),
                beta=torch.sigmoid(beta_logit).to(dt), A=A, S0=S0, cu_seqlens=cu.to(device))


def _taps_and_states(w: Workload, width: int, g, B: int, device, dt):
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    scale = 1.0 / float(width) ** 0.5
    taps = tuple(torch.randn(w.H, d, width, **f32).mul_(scale) for d in (w.dk, w.dk, w.dv))
    states = tuple(torch.randn(B, width - 1, w.H, d, **f32).to(dt) for d in (w.dk, w.dk, w.dv))
    return taps, states


def make_layer_inputs(w: Workload, width: int, device="cpu", T: int | None = None):
    """Raw layer inputs of a prefill workload for the prologue path: q, k, v
    (not normalized), z, beta, A, S0, taps (wq, wk, wv) and conv states
    (sq, sk, sv)."""
    T = w.T if T is None else int(T)
    g = _gen(w.seed, device)
    dt = torch_dtype(w.dtype)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    q = torch.randn(w.B, T, w.H, w.dk, **f32)
    k = torch.randn(w.B, T, w.H, w.dk, **f32)
    v = torch.randn(w.B, T, w.H, w.dv, **f32)
    beta_logit = torch.randn(w.B, T, w.H, **f32)
    z = torch.randn(w.B, T, w.H, w.dk, **f32)
    if w.z_mean:
        z.add_(w.z_mean)
    A = torch.rand(w.H, **f32).mul_(2.0).sub_(1.0)
    S0 = None
    if w.s0_std is not None:
        S0 = torch.randn(w.B, w.H, w.dk, w.dv, **f32).mul_(w.s0_std)
    (wq, wk, wv), (sq, sk, sv) = _taps_and_states(w, width, g, w.B, device, dt)
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), z=z.to(dt),
                beta=torch.sigmoid(beta_logit).to(dt), A=A, S0=S0,
                wq=wq, wk=wk, wv=wv, sq=sq, sk=sk, sv=sv)


def make_layer_decode_inputs(w: Workload, width: int, device="cpu", steps: int | None = None):
    """Per-step raw decode inputs (leading [steps] axis, q, k not normalized),
    A, a zero S, taps and conv states."""
    steps = w.steps if steps is None else int(steps)
    g = _gen(w.seed, device)
    dt = torch_dtype(w.dtype)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    q = torch.randn(steps, w.B, w.H, w.dk, **f32)
    k = torch.randn(steps, w.B, w.H, w.dk, **f32)
    v = torch.randn(steps, w.B, w.H, w.dv, **f32)
    beta_logit = torch.randn(steps, w.B, w.H, **f32)
    z = torch.randn(steps, w.B, w.H, w.dk, **f32)
    if w.z_mean:
        z.add_(w.z_mean)
    A = torch.rand(w.H, **f32).mul_(2.0).sub_(1.0)
    S = torch.zeros(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=device)
    (wq, wk, wv), (sq, sk, sv) = _taps_and_states(w, width, g, w.B, device, dt)
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), z=z.to(dt),
                beta=torch.sigmoid(beta_logit).to(dt), A=A, S=S,
                wq=wq, wk=wk, wv=wv, sq=sq, sk=sk, sv=sv)


def make_cotangents(w: Workload, device="cpu", T: int | None = None, with_dST: bool = True):
    """dO [B, T, H, dv] (run dtype) and dL/dS_T [B, H, dk, dv] (fp32, or None)
    for a prefill workload, from the seed + 1000 stream."""
    T = w.T if T is None else int(T)
    g = _gen(w.seed + 1000, device)
    f32 = dict(dtype=torch.float32, device=device, generator=g)
    dO = torch.randn(w.B, T, w.H, w.dv, **f32).to(torch_dtype(w.dtype))
    dST = torch.randn(w.B, w.H, w.dk, w.dv, **f32) if with_dST else None
    return dO, dST
