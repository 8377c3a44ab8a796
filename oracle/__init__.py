"""fp64 CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library and its Python
binding never import, link or call it, and it shares no code with them.

The arithmetic lives in ``kda_oracle.c`` (a plain sequential fp64 loop over
the KDA recurrence and its bounded decay gate; see that file's header for the
page sections it follows).  This module only marshals numpy arrays into it.

Parity status of each function (what pins it, see ``tests/test_oracle_pins.py``):
  gate      -- pinned: exact special values (z=0, +-inf), range [-5, 0],
               agreement with scipy's logistic function.
  prefill   -- pinned: brute-force product expansion, closed forms (beta=0,
               T=1, dk=1), overwrite, capacity, an independent fp64 chunked
               model, split / linearity / independence invariants.
  decode_step -- pinned: T single steps equal one prefill over T, T=1 closed form.
  prefill_bwd -- pinned: central finite differences of the (pinned) forward
               on every input element of small cases, T = 0 and beta = 0
               special cases, a planted-mistake battery.
  prefill_conv, decode_step_conv -- the prologue of ``oracle/prologue.py``
               (short convolutions, q/k normalization) followed by the pinned
               recurrence; see that module for the readings and pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

__all__ = ["build", "gate", "prefill", "prefill_bwd", "decode_step", "prefill_conv",
           "decode_step_conv", "max_threads"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc -O2 (no fast-math) and OpenMP."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.kda_oracle_f64.restype = ctypes.c_int
    lib.kda_oracle_f64.argtypes = [i64, i64, i64, i64, i64,
                                   dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                   ctypes.c_int]
    lib.kda_oracle_gate_f64.restype = None
    lib.kda_oracle_gate_f64.argtypes = [i64, dp, ctypes.c_double, dp]
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    lib.kda_oracle_bwd_f64.restype = ctypes.c_int
    lib.kda_oracle_bwd_f64.argtypes = [i64, i64, i64, i64, i64] + [dp] * 16 + [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # KDA_ORACLE_LIB: another build of kda_oracle.c to run (the sanitizer test
    # runs the pin tests against an instrumented build)
    if os.environ.get("KDA_ORACLE_LIB"):
        _lib = _bind(os.environ["KDA_ORACLE_LIB"])
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build(force=True)
    _lib = _bind(_LIB_PATH)
    return _lib


def load_variant(path: str):
    """Bind another build of kda_oracle.c (used by the test that plants
    mistakes in a copy of the oracle to show the pins catch them)."""
    return _bind(path)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def gate(z, A: float, lib=None) -> np.ndarray:
    """g = -5 * sigmoid(e^A * z), elementwise, fp64."""
    z = _f64(z)
    out = np.empty_like(z)
    (lib or _load()).kda_oracle_gate_f64(z.size, _ptr(z), float(A), _ptr(out))
    return out


def prefill(q, k, v, z, beta, A, S0=None, threads: int | None = None, lib=None):
    """Run the KDA recurrence over all T tokens.

    Shapes: q, k, z [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]; A [H];
    S0 [B,H,dk,dv] or None (zeros).  Inputs are upcast exactly to fp64.
    Returns (o [B,T,H,dv], S_T [B,H,dk,dv]) in fp64.
    """
    q, k, v, z, beta, A = (_f64(x) for x in (q, k, v, z, beta, A))
    if q.ndim != 4:
        raise ValueError("q must be [B,T,H,dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or z.shape != q.shape:
        raise ValueError("k and z must match q's shape")
    if v.shape != (B, T, H, dv) or beta.shape != (B, T, H) or A.shape != (H,):
        raise ValueError("bad v / beta / A shape")
    s0 = None
    if S0 is not None:
        s0 = _f64(S0)
        if s0.shape != (B, H, dk, dv):
            raise ValueError("S0 must be [B,H,dk,dv]")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    S_T = np.zeros((B, H, dk, dv), dtype=np.float64)
    n = threads if threads is not None else (os.cpu_count() or 1)
    n = max(1, min(int(n), max(1, B * H)))
    rc = (lib or _load()).kda_oracle_f64(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(z), _ptr(beta), _ptr(A), _ptr(s0),
                                _ptr(o), _ptr(S_T), n)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_f64 failed with code {rc}")
    return o, S_T


def prefill_bwd(q, k, v, z, beta, A, S0, dO, dST=None, threads: int | None = None, lib=None):
    """Gradients of L through the recurrence, given dO = dL/do [B,T,H,dv] and
    dST = dL/dS_T [B,H,dk,dv] (None = 0).  Returns a dict with dq, dk, dz
    [B,T,H,dk], dv [B,T,H,dv], dbeta [B,T,H], dA [H], dS0 [B,H,dk,dv] (fp64)."""
    q, k, v, z, beta, A, dO = (_f64(x) for x in (q, k, v, z, beta, A, dO))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    s0 = None if S0 is None else _f64(S0)
    dst = None if dST is None else _f64(dST)
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)),
           "dv": np.zeros((B, T, H, dv)), "dz": np.zeros((B, T, H, dk)),
           "dbeta": np.zeros((B, T, H)), "dA": np.zeros((H,)), "dS0": np.zeros((B, H, dk, dv))}
    n = threads if threads is not None else (os.cpu_count() or 1)
    n = max(1, min(int(n), max(1, B * H)))
    rc = (lib or _load()).kda_oracle_bwd_f64(
        B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(beta), _ptr(A), _ptr(s0),
        _ptr(dO), _ptr(dst), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dz"]),
        _ptr(out["dbeta"]), _ptr(out["dA"]), _ptr(out["dS0"]), n)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_bwd_f64 failed with code {rc}")
    return out


def decode_step(q, k, v, z, beta, A, S, threads: int | None = None):
    """One recurrent step.  q, k, z [B,H,dk]; v [B,H,dv]; beta [B,H]; S [B,H,dk,dv].
    Returns (o [B,H,dv], S_new [B,H,dk,dv]) in fp64."""
    q, k, v, z, beta = (_f64(x)[:, None] for x in (q, k, v, z, beta))
    o, S_new = prefill(q, k, v, z, beta, A, S, threads=threads)
    return o[:, 0], S_new


def prefill_conv(q, k, v, z, beta, A, wq, wk, wv, conv_state=None, act="none", eps=1e-6,
                 S0=None, threads: int | None = None):
    """Prologue + recurrence over a segment of T tokens.

    q, k, v raw (pre-convolution) [B,T,H,d]; wq, wk [H,dk,W], wv [H,dv,W];
    conv_state None or (state_q, state_k, state_v), each [B,W-1,H,d].
    Returns (o, S_T, (state_q, state_k, state_v)) in fp64."""
    from .prologue import conv_norm
    sq, sk, sv = conv_state if conv_state is not None else (None, None, None)
    qh, kh, vc, states = conv_norm(q, k, v, wq, wk, wv, sq, sk, sv, act, eps)
    o, S_T = prefill(qh, kh, vc, z, beta, A, S0, threads=threads)
    return o, S_T, states


def decode_step_conv(q, k, v, z, beta, A, wq, wk, wv, conv_state, S, act="none", eps=1e-6):
    """One token through prologue and recurrence.  q, k, z [B,H,dk]; v [B,H,dv];
    beta [B,H]; conv_state (state_q, state_k, state_v) each [B,W-1,H,d]; S [B,H,dk,dv].
    Returns (o [B,H,dv], S_new, new conv states)."""
    o, S_new, states = prefill_conv(*(_f64(x)[:, None] for x in (q, k, v, z, beta)), A,
                                    wq, wk, wv, conv_state, act, eps, S)
    return o[:, 0], S_new, states
