"""Shared helpers for the GPU parity tests."""
import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def slice_relerr(x, ref, head_axis: int) -> float:
    """Max over (b, h) slices of max|x - ref| / max|ref| (normwise per slice).
    x, ref have a leading batch axis and the head axis at ``head_axis``."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for b in range(ref.shape[0]):
        for h in range(ref.shape[head_axis]):
            xs = np.take(x[b], h, axis=head_axis - 1)
            rs = np.take(ref[b], h, axis=head_axis - 1)
            den = np.max(np.abs(rs)) if rs.size else 0.0
            num = np.max(np.abs(xs - rs)) if rs.size else 0.0
            worst = max(worst, num / den if den > 0 else num)
    return float(worst)


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


def gpu_prefill(kda, g, chunk, **kw):
    o, S_T = kda.prefill(g["q"], g["k"], g["v"], g["z"], g["beta"], g["A"], g["S0"],
                         chunk=chunk, **kw)
    torch.cuda.synchronize()
    return o, S_T
