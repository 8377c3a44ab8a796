"""Independent fp64 models used to pin the oracle (CPU, numpy).

None of these calls the oracle; each computes a result that the KDA recurrence
must reproduce by a route other than the oracle's sequential loop:

  brute_force   -- explicit dk x dk transition matrices
                   P_t = (I - beta_t k_t k_t^T) Diag(alpha_t), multiplied out
                   term by term (each summand of the unrolled recurrence is
                   formed on its own).
  chunked       -- the chunk-parallel (WY / UT-transform) form of the same
                   recurrence: within a chunk, the pairwise decayed key
                   products give a unit lower-triangular system whose inverse
                   maps the chunk's values to the state corrections.
  decay         -- alpha = exp(-5 * logistic(e^A z)) through scipy's logistic.

The recurrence and gate they model are those of "Kimi K3 Open Weights: What Is
Actually New", section 1 (the single-head state equation and the bounded
decay-gate equation).
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit

G_MIN = -5.0


def decay(z: np.ndarray, A: float) -> np.ndarray:
    """alpha = e^g with g = g_min * logistic(e^A * z), through scipy."""
    return np.exp(G_MIN * expit(np.exp(A) * np.asarray(z, dtype=np.float64)))


def log_decay(z: np.ndarray, A: float) -> np.ndarray:
    return G_MIN * expit(np.exp(A) * np.asarray(z, dtype=np.float64))


def brute_force(q, k, v, z, beta, A, S0=None):
    """Unrolled recurrence for one batch entry at a time.

    S_t = (P_t ... P_1) S0 + sum_{s<=t} (P_t ... P_{s+1}) beta_s k_s v_s^T,
    o_t = S_t^T q_t.  Shapes as the oracle's.  O(T^2 dk^3): tiny cases only."""
    q, k, v, z, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, z, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)[b, h]
            P = [(I - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h]))
                 @ np.diag(decay(z[b, t, h], A[h])) for t in range(T)]
            for t in range(T):
                prod = I.copy()
                for s in range(t, -1, -1):
                    prod = prod @ P[s]
                St = prod @ s0
                for s in range(t + 1):
                    tail = I.copy()
                    for r in range(t, s, -1):
                        tail = tail @ P[r]
                    St = St + tail @ (beta[b, s, h] * np.outer(k[b, s, h], v[b, s, h]))
                o[b, t, h] = St.T @ q[b, t, h]
                if t == T - 1:
                    S_T[b, h] = St
            if T == 0:
                S_T[b, h] = s0
    return o, S_T


def chunked(q, k, v, z, beta, A, S0=None, chunk=16):
    """Chunk-parallel form, fp64.

    Per chunk of length n with entering state S and in-chunk cumulative
    log-decay G_r = sum_{s<=r} g_s (per key channel):
      L[r,s] = beta_r sum_d k_r[d] k_s[d] e^{G_r[d]-G_s[d]}     (s <  r)
      P[r,s] =        sum_d q_r[d] k_s[d] e^{G_r[d]-G_s[d]}     (s <= r)
      T  = (I + L)^{-1}
      W  = T diag(beta) (K * e^G),   U~ = T diag(beta) V
      U  = U~ - W S
      O  = (Q * e^G) S + P U
      S <- e^{G_n} * S + (K * e^{G_n - G})^T U
    """
    q, k, v, z, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, z, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)[b, h]
            for c0 in range(0, T, chunk):
                sl = slice(c0, min(T, c0 + chunk))
                Q, K, V, Z, be = q[b, sl, h], k[b, sl, h], v[b, sl, h], z[b, sl, h], beta[b, sl, h]
                n = Q.shape[0]
                G = np.cumsum(log_decay(Z, A[h]), axis=0)
                D = np.exp(G[:, None, :] - G[None, :, :])        # [r, s, d]
                tri = np.tril(np.ones((n, n)), -1)
                L = be[:, None] * np.einsum("rd,sd,rsd->rs", K, K, np.where(tri[..., None] > 0, D, 0.0))
                Pm = np.einsum("rd,sd,rsd->rs", Q, K,
                               np.where(np.tril(np.ones((n, n)))[..., None] > 0, D, 0.0))
                Tm = np.linalg.inv(np.eye(n) + L)
                W = Tm @ (be[:, None] * K * np.exp(G))
                Ut = Tm @ (be[:, None] * V)
                U = Ut - W @ S
                o[b, sl, h] = (Q * np.exp(G)) @ S + Pm @ U
                S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ U
            S_T[b, h] = S
    return o, S_T


def chunked_bwd(q, k, v, z, beta, A, S0, dO, dST=None, chunk=16):
    """Chunk-parallel reverse mode, fp64: the adjoint of ``chunked``, chunk by
    chunk in reverse, carrying dS between chunks.  A model of the training form
    (what a chunked GPU backward computes), checked against the step-by-step
    adjoint oracle.  Per chunk, with the forward quantities of ``chunked`` and
    Kh = K * e^{G_n - G}, Q^ = Q * e^G, K^ = K * e^G:
      dU  = P^T dO + Kh dS'            dS  = Q^^T dO + e^{G_n} * dS' - W^T dU
      dP  = tril(dO U^T)                dW  = -dU S^T
      dT  = dW (beta K^)^T + dU (beta V)^T,  dL = -T^T dT T^T (strictly lower)
    then the gradients of the decayed products flow to q, k, beta and to the
    cumulative log-decay G, whose reverse cumulative sum is dg; the gate gives
    dz and dA.  Returns the dict of ``oracle.prefill_bwd``."""
    q, k, v, z, beta, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, z, beta, dO))
    A = np.asarray(A, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dz": np.zeros_like(z), "dbeta": np.zeros_like(beta), "dA": np.zeros(H),
           "dS0": np.zeros((B, H, dk, dv))}
    for b in range(B):
        for h in range(H):
            c = np.exp(A[h])
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)[b, h]
            starts = list(range(0, T, chunk))
            S_in = []
            # forward, keeping each chunk's entering state
            for c0 in starts:
                sl = slice(c0, min(T, c0 + chunk))
                S_in.append(S.copy())
                _, S = _chunk_forward(q[b, sl, h], k[b, sl, h], v[b, sl, h], z[b, sl, h],
                                      beta[b, sl, h], A[h], S)
            dS = np.zeros((dk, dv)) if dST is None else np.array(dST, np.float64)[b, h]
            for ci in range(len(starts) - 1, -1, -1):
                sl = slice(starts[ci], min(T, starts[ci] + chunk))
                g = _chunk_backward(q[b, sl, h], k[b, sl, h], v[b, sl, h], z[b, sl, h],
                                    beta[b, sl, h], A[h], S_in[ci], dO[b, sl, h], dS)
                dS = g["dS"]
                out["dq"][b, sl, h] = g["dq"]
                out["dk"][b, sl, h] = g["dk"]
                out["dv"][b, sl, h] = g["dv"]
                out["dz"][b, sl, h] = g["dz"]
                out["dbeta"][b, sl, h] = g["dbeta"]
                out["dA"][h] += g["dA"]
            out["dS0"][b, h] = dS
    return out


def _chunk_quantities(Q, K, V, Z, be, A, S):
    n = Q.shape[0]
    G = np.cumsum(log_decay(Z, A), axis=0)
    D = np.exp(G[:, None, :] - G[None, :, :])
    strict = np.tril(np.ones((n, n)), -1)
    lower = np.tril(np.ones((n, n)))
    Akk = np.einsum("rd,sd,rsd->rs", K, K, D) * strict
    Pm = np.einsum("rd,sd,rsd->rs", Q, K, D) * lower
    L = be[:, None] * Akk
    Tm = np.linalg.inv(np.eye(n) + L)
    KG = K * np.exp(G)
    QG = Q * np.exp(G)
    W = Tm @ (be[:, None] * KG)
    Ut = Tm @ (be[:, None] * V)
    U = Ut - W @ S
    Gn = G[-1]
    Kh = K * np.exp(Gn[None, :] - G)
    return dict(G=G, D=D, strict=strict, lower=lower, Akk=Akk, Pm=Pm, Tm=Tm, KG=KG, QG=QG, W=W,
                U=U, Gn=Gn, Kh=Kh)


def _chunk_forward(Q, K, V, Z, be, A, S):
    x = _chunk_quantities(Q, K, V, Z, be, A, S)
    O = x["QG"] @ S + x["Pm"] @ x["U"]
    S_new = np.exp(x["Gn"])[:, None] * S + x["Kh"].T @ x["U"]
    return O, S_new


def _chunk_backward(Q, K, V, Z, be, A, S, dO, dSp):
    x = _chunk_quantities(Q, K, V, Z, be, A, S)
    G, D, Tm, KG, QG, W, U, Gn, Kh = (x[n] for n in ("G", "D", "Tm", "KG", "QG", "W", "U", "Gn",
                                                     "Kh"))
    Gamma_n = np.exp(Gn)
    dU = x["Pm"].T @ dO + Kh @ dSp
    dS = QG.T @ dO + Gamma_n[:, None] * dSp - W.T @ dU
    dPm = (dO @ U.T) * x["lower"]
    dQG = dO @ S.T
    dKh = U @ dSp.T
    dGn = (dSp * S).sum(axis=1) * Gamma_n
    dW = -dU @ S.T
    dTm = dW @ (be[:, None] * KG).T + dU @ (be[:, None] * V).T
    dBKG = Tm.T @ dW
    dBV = Tm.T @ dU
    dKG = be[:, None] * dBKG
    dV = be[:, None] * dBV
    dbe = (dBKG * KG).sum(axis=1) + (dBV * V).sum(axis=1)
    dL = -(Tm.T @ dTm @ Tm.T) * x["strict"]
    dbe += (dL * x["Akk"]).sum(axis=1)
    dAkk = be[:, None] * dL
    dQ = np.einsum("rs,sd,rsd->rd", dPm, K, D) + dQG * np.exp(G)
    dK = (np.einsum("rs,sd,rsd->rd", dAkk, K, D) + np.einsum("rs,rd,rsd->sd", dAkk, K, D)
          + np.einsum("rs,rd,rsd->sd", dPm, Q, D) + dKG * np.exp(G) + dKh * np.exp(Gn[None, :] - G))
    tk = np.einsum("rs,rd,sd,rsd->rsd", dAkk, K, K, D)
    tq = np.einsum("rs,rd,sd,rsd->rsd", dPm, Q, K, D)
    dG = tk.sum(axis=1) - tk.sum(axis=0) + tq.sum(axis=1) - tq.sum(axis=0)
    dG += dQG * QG + dKG * KG - dKh * Kh
    dGn = dGn + (dKh * Kh).sum(axis=0)
    dG[-1] += dGn
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    xz = np.exp(A) * Z
    sig = expit(xz)
    dx = dg * G_MIN * sig * (1.0 - sig)
    return {"dS": dS, "dq": dQ, "dk": dK, "dv": dV, "dbeta": dbe, "dz": dx * np.exp(A),
            "dA": float(np.sum(dx * xz))}


def relerr(x, ref) -> float:
    """max |x - ref| / max |ref| (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)
