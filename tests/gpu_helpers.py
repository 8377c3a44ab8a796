"""Shared helpers for the GPU parity tests."""
import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


FP32_MIN_NORMAL = 2.0 ** -126


def slice_relerr(x, ref, head_axis: int) -> float:
    """Max over (b, h) slices of max|x - ref| / max(max|ref|, 2^-126)
    (normwise per slice).  The floor only matters for a slice whose whole
    reference lies below fp32's normal range, where a GPU result, fp32 at
    best, cannot carry relative precision; there the error is absolute,
    relative to 2^-126.  x, ref have a leading batch axis and the head axis at
    ``head_axis``."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[head_axis]):
            xs = np.take(x[b], h, axis=head_axis - 1)
            rs = np.take(ref[b], h, axis=head_axis - 1)
            den = max(np.max(np.abs(rs)), FP32_MIN_NORMAL) if rs.size else FP32_MIN_NORMAL
            num = np.max(np.abs(xs - rs)) if rs.size else 0.0
            worst = max(worst, num / den)
    return float(worst)


def elem_relerr(x, ref, head_axis: int, floor: float = 1e-6):
    """Elementwise diagnostic (reported, not gated): per (b, h) slice, the
    relative error of every element, |x - ref| / max(|ref|, floor * max|ref|).
    Returns (max, 99.9th percentile, fraction of elements above 2e-2), each
    the worst over slices."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = [0.0, 0.0, 0.0]
    for b in range(ref.shape[0]):
        for h in range(ref.shape[head_axis]):
            xs = np.take(x[b], h, axis=head_axis - 1).ravel()
            rs = np.take(ref[b], h, axis=head_axis - 1).ravel()
            if rs.size == 0:
                continue
            m = np.max(np.abs(rs))
            if m == 0:
                continue
            r = np.abs(xs - rs) / np.maximum(np.abs(rs), floor * m)
            worst[0] = max(worst[0], float(np.max(r)))
            worst[1] = max(worst[1], float(np.percentile(r, 99.9)))
            worst[2] = max(worst[2], float(np.mean(r > 2e-2)))
    return tuple(worst)


def row_relerr(x, ref, floor: float = 1e-3):
    """Token-row diagnostic (reported, not gated) for [B, T, H, d] outputs:
    per (b, t, h) row, max|x - ref| / max(max|ref row|, floor * max|ref|
    over the (b, h) slice).  Returns (max, 99.9th percentile) over rows."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return (0.0, 0.0)
    num = np.max(np.abs(x - ref), axis=-1)                       # [B, T, H]
    den = np.max(np.abs(ref), axis=-1)
    scale = np.max(den, axis=1, keepdims=True)                   # per (b, h)
    r = num / np.maximum(np.maximum(den, floor * scale), 1e-300)
    return (float(np.max(r)), float(np.percentile(r, 99.9)))


def fmt_elem(e, rows=None) -> str:
    s = f"elementwise max {e[0]:.2e} p99.9 {e[1]:.2e} frac>2e-2 {e[2]:.2e}"
    if rows is not None:
        s += f"; token rows max {rows[0]:.2e} p99.9 {rows[1]:.2e}"
    return s


def diag(x, ref) -> str:
    """Both diagnostics of an output [B, T, H, d] against its reference."""
    return fmt_elem(elem_relerr(x, ref, 2), row_relerr(x, ref))


def host(t):
    return None if t is None else t.detach().float().cpu().numpy()


def to_dev(inp, dev):
    return {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}


def oracle_prefill(inp, heads=None, T=None):
    """Oracle on host copies of the inputs, optionally for a subset of heads
    and a prefix of the tokens."""
    def sel(t, axis):
        if t is None:
            return None
        if T is not None and axis == 2:
            t = t[:, :T]
        if heads is not None:
            idx = torch.as_tensor(heads, device=t.device)
            t = torch.index_select(t, axis, idx)
        return host(t)
    q, k, v, z = (sel(inp[n], 2) for n in ("q", "k", "v", "z"))
    beta = sel(inp["beta"], 2)
    A = host(inp["A"]) if heads is None else host(inp["A"])[heads]
    S0 = sel(inp["S0"], 1)
    return oracle.prefill(q, k, v, z, beta, A, S0)


def oracle_prefill_chained(inp, heads, seg: int = 1 << 17):
    """Oracle over the full length for a few heads, run segment by segment
    with the state carried from one segment into the next (the split property
    of the recurrence, pinned on the oracle itself), so host memory holds one
    segment's fp64 inputs at a time.  Returns (o as float32 [B, T, len(heads),
    dv], S_T fp64)."""
    idx = None
    T = inp["q"].shape[1]
    A = host(inp["A"])[heads]
    S = None
    if inp["S0"] is not None:
        S = host(torch.index_select(inp["S0"], 1, torch.as_tensor(heads, device=inp["S0"].device)))
    outs = []
    for t0 in range(0, T, seg):
        part = []
        for n in ("q", "k", "v", "z", "beta"):
            t = inp[n]
            if idx is None:
                idx = torch.as_tensor(heads, device=t.device)
            part.append(host(torch.index_select(t[:, t0:t0 + seg], 2, idx)))
        o, S = oracle.prefill(*part, A, S)
        outs.append(o.astype(np.float32))
    return np.concatenate(outs, axis=1), S


def gpu_prefill(kda, g, chunk, **kw):
    o, S_T = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], g["S0"],
                         chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, S_T
