"""fp64 CPU oracle for the KDA prologue -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module; the GPU library never does.

"Kimi K3 Open Weights: What Is Actually New", section 1 ("Kimi Delta Attention
is a real new kernel family") lists short convolutions and Q/K normalization
among the prefill steps ahead of the decay products and chunk interactions,
and says one-token decode keeps a convolution state next to the recurrent
state; the same page's section "Why '104B active' still understates the
systems problem" counts a short-convolution state per request and layer.  The
page gives neither the width, an activation nor the normalization's guard, so
this module takes these readings (each one a parameter where a choice exists):

  * q, k and v each pass through their own causal depthwise convolution over
    tokens: channel c of token t is sum_{j<W} w[c, j] * x[t - (W-1) + j][c],
    so tap W-1 weighs the current token.  Weights are [H, d, W].
  * Tokens before the first one come from the convolution state: the last
    W-1 raw (pre-convolution) inputs of the same sequence, oldest first,
    [B, W-1, H, d]; a fresh sequence starts from zeros.  After the segment
    the state holds the last W-1 raw inputs of state + segment.
  * An optional SiLU, x * logistic(x), follows the convolution (act="silu");
    the default applies none.
  * q and k are then L2-normalized per token and head over the key channels:
    x / sqrt(sum x^2 + eps).  v is not normalized.
  * The decay input z and the write strength beta bypass the prologue.

Parity status (tests/test_oracle_prologue.py):
  short_conv  -- pinned: single channels against numpy.convolve, delta taps
                 (identity, pure delay through the state), state carry over a
                 split segment, linearity in x and in w.
  silu        -- pinned: scipy's logistic function, exact values at 0.
  l2norm      -- pinned: closed form on a 3-4-5 vector, unit norm, scale
                 invariance, zero vector with eps > 0.
  conv_norm / prefill_conv / decode_step_conv -- compositions of the pinned
                 parts with the pinned recurrence; decode steps are pinned
                 against one prefill over the same tokens.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def silu(x):
    """x * logistic(x) in fp64."""
    x = _f64(x)
    return x * expit(x)


def short_conv(x, w, state=None, act: str = "none"):
    """Causal depthwise convolution of one tensor over its token axis.

    x [B, T, H, d]; w [H, d, W]; state [B, W-1, H, d] or None (zeros).
    Returns (y [B, T, H, d], new_state [B, W-1, H, d]).  The new state holds
    raw inputs, so carrying it into the next segment continues the sequence.
    """
    x, w = _f64(x), _f64(w)
    B, T, H, d = x.shape
    W = w.shape[-1]
    if w.shape != (H, d, W) or W < 1:
        raise ValueError("w must be [H, d, W] with W >= 1")
    if state is None:
        state = np.zeros((B, W - 1, H, d))
    state = _f64(state)
    if state.shape != (B, W - 1, H, d):
        raise ValueError("state must be [B, W-1, H, d]")
    # the raw sequence, W-1 earlier tokens first: xp[W-1 + t] = x[t]
    xp = np.concatenate([state, x], axis=1)
    y = np.zeros_like(x)
    for j in range(W):
        y += w[None, None, :, :, j] * xp[:, j:j + T]
    if act == "silu":
        y = silu(y)
    elif act != "none":
        raise ValueError("act must be 'none' or 'silu'")
    new_state = xp[:, xp.shape[1] - (W - 1):]
    return y, np.ascontiguousarray(new_state)


def l2norm(x, eps: float):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def conv_norm(q, k, v, wq, wk, wv, state_q=None, state_k=None, state_v=None,
              act: str = "none", eps: float = 1e-6):
    """The prologue: convolve q, k, v, then L2-normalize q and k.

    Returns (q_hat, k_hat, v_conv, (state_q, state_k, state_v)) in fp64."""
    qc, sq = short_conv(q, wq, state_q, act)
    kc, sk = short_conv(k, wk, state_k, act)
    vc, sv = short_conv(v, wv, state_v, act)
    return l2norm(qc, eps), l2norm(kc, eps), vc, (sq, sk, sv)
