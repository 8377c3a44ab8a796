"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: exact special
values, closed forms, a brute-force expansion, an independent chunk-parallel
model, and structural invariants of the KDA recurrence ("Kimi K3 Open Weights:
What Is Actually New", section 1, state equation and bounded gate equation).
Shapes use dk != dv wherever a transposed state or a decay applied to the wrong
side would otherwise go unnoticed.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.kda_pins import brute_force, chunked, decay, log_decay, relerr

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_page_constants.json")


def _rand_inputs(rng, B, T, H, dk, dv, z_mean=0.0, beta_range=(0.0, 1.0), unit=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk)) + z_mean
    beta = rng.uniform(*beta_range, size=(B, T, H))
    A = rng.uniform(-1, 1, size=(H,))
    return q, k, v, z, beta, A


# ---------------------------------------------------------------- gate ----

def test_gate_special_values():
    g = oracle.gate(np.array([0.0, 1e4, -1e4, np.inf, -np.inf]), 0.37)
    assert g[0] == -2.5                      # sigma(0) = 1/2 for any A
    assert g[1] == -5.0 and g[3] == -5.0     # saturates at g_min
    assert g[2] == 0.0 and g[4] == 0.0       # -> -0: alpha = 1 exactly
    assert math.exp(g[2]) == 1.0


def test_gate_matches_library_logistic_and_range():
    rng = np.random.default_rng(1)
    z = rng.standard_normal(4096) * 4
    for A in (-1.0, -0.3, 0.0, 0.8, 1.0):
        g = oracle.gate(z, A)
        ref = -5.0 * expit(np.exp(A) * z)
        np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-300)
        assert np.all(g <= 0.0) and np.all(g >= -5.0)
        order = np.argsort(z)
        assert np.all(np.diff(g[order]) <= 0.0)   # decreasing in z (e^A > 0)


def test_gate_extreme_scales():
    """Far outside the usual A: e^A underflowing to 0 gives sigma(0) = 1/2 for
    every finite z (g = g_min / 2); a large e^A saturates the logistic to
    g_min or 0 except right at z = 0 -- as the library logistic says."""
    z = np.array([-30.0, -1.0, -1e-3, 0.0, 1e-3, 1.0, 30.0])
    assert np.all(oracle.gate(z, -800.0) == -2.5)          # e^A = 0 exactly in fp64
    g = oracle.gate(z, -100.0)                              # e^A = 3.7e-44
    np.testing.assert_allclose(g, -5.0 * expit(np.exp(-100.0) * z), rtol=1e-15)
    assert np.all(np.abs(g + 2.5) < 1e-40)
    g = oracle.gate(z, 4.0)                                 # e^A = 54.6
    np.testing.assert_allclose(g, -5.0 * expit(np.exp(4.0) * z), rtol=1e-14, atol=1e-300)
    assert g[0] == 0.0 and g[-1] == -5.0 and g[3] == -2.5


def test_page_range_claim():
    """g_min = -5 bounds a 16-token log-decay window by -80, and e^80 fits bf16."""
    c = json.load(open(GOLDEN))
    gmin = c["g_min"]["value"]
    tile = c["rescale_tile_tokens"]["value"]
    bound = c["reciprocal_exponent_bound"]["value"]
    assert gmin * tile == -bound
    assert math.exp(bound) < c["bf16_max"]["value"]
    # the oracle's gate never leaves [g_min, 0], so no window can pass -80
    z = np.full(tile, 1e6)
    g = oracle.gate(z, 1.0)
    assert np.all(g == gmin)
    assert g.sum() == -bound
    assert math.exp(-g.sum()) < c["bf16_max"]["value"]


# ----------------------------------------------------- closed forms ----

def test_beta_zero_is_pure_channelwise_decay():
    """beta = 0: S_T = Diag(prod alpha) S0, o_t = S0^T (prod_{s<=t} alpha_s * q_t).
    Pins that the decay scales the KEY rows of S (dk != dv)."""
    rng = np.random.default_rng(2)
    B, T, H, dk, dv = 2, 9, 3, 5, 7
    q, k, v, z, _, A = _rand_inputs(rng, B, T, H, dk, dv)
    beta = np.zeros((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    for b in range(B):
        for h in range(H):
            cum = np.ones(dk)
            for t in range(T):
                cum = cum * decay(z[b, t, h], A[h])
                np.testing.assert_allclose(o[b, t, h], S0[b, h].T @ (cum * q[b, t, h]),
                                           rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(S_T[b, h], cum[:, None] * S0[b, h], rtol=1e-13,
                                       atol=1e-15)


def test_single_token_closed_form():
    """T = 1: o = S0^T(alpha*q) + beta (q.k) (v - S0^T(alpha*k)).  Pins that the
    read uses the UPDATED state (o reads S_1, not S_0)."""
    rng = np.random.default_rng(3)
    B, H, dk, dv = 3, 2, 6, 4
    q, k, v, z, beta, A = _rand_inputs(rng, B, 1, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    for b in range(B):
        for h in range(H):
            a = decay(z[b, 0, h], A[h])
            qq, kk, vv, bb, s0 = q[b, 0, h], k[b, 0, h], v[b, 0, h], beta[b, 0, h], S0[b, h]
            exp_o = s0.T @ (a * qq) + bb * (qq @ kk) * (vv - s0.T @ (a * kk))
            np.testing.assert_allclose(o[b, 0, h], exp_o, rtol=1e-13, atol=1e-14)
            exp_S = a[:, None] * s0 + np.outer(kk, bb * (vv - s0.T @ (a * kk)))
            np.testing.assert_allclose(S_T[b, h], exp_S, rtol=1e-13, atol=1e-14)
    # zero state: o = beta (q.k) v
    o2, _ = oracle.prefill(q, k, v, z, beta, A, None)
    exp = beta[..., None] * np.einsum("bthd,bthd->bth", q, k)[..., None] * v
    np.testing.assert_allclose(o2, exp, rtol=1e-13, atol=1e-15)


def test_scalar_key_is_gated_ema():
    """dk = 1: S_t = (1 - beta k^2) alpha S_{t-1} + beta k v_t (a gated EMA per
    value column), o_t = S_t q_t."""
    rng = np.random.default_rng(4)
    T, dv = 40, 3
    q, k, v, z, beta, A = _rand_inputs(rng, 1, T, 1, 1, dv, unit=False)
    o, S_T = oracle.prefill(q, k, v, z, beta, A, None)
    s = np.zeros(dv)
    for t in range(T):
        a = math.exp(-5.0 * expit(math.exp(A[0]) * z[0, t, 0, 0]))
        kk = k[0, t, 0, 0]
        s = (1.0 - beta[0, t, 0] * kk * kk) * a * s + beta[0, t, 0] * kk * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], s * q[0, t, 0, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S_T[0, 0, 0], s, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------ delta rule ----

@pytest.mark.parametrize("random_key", [False, True])
def test_overwrite_same_key(random_key):
    """alpha = 1 (z = -1e4), beta = 1, the same unit key written twice: reading
    with that key returns v2, not v1 + v2 (the delta rule overwrites)."""
    rng = np.random.default_rng(5)
    dk, dv = 8, 5
    if random_key:
        key = rng.standard_normal(dk)
        key /= np.linalg.norm(key)
    else:
        key = np.eye(dk)[0]
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    q = np.stack([key, key])[None, :, None]
    k = q.copy()
    v = np.stack([v1, v2])[None, :, None]
    z = np.full((1, 2, 1, dk), -1e4)
    beta = np.ones((1, 2, 1))
    o, S_T = oracle.prefill(q, k, v, z, beta, np.array([0.4]), None)
    tol = 0.0 if not random_key else 1e-14
    assert np.max(np.abs(o[0, 1, 0] - v2)) <= tol * np.max(np.abs(v2)) + tol
    assert np.max(np.abs(o[0, 0, 0] - v1)) <= tol * np.max(np.abs(v1)) + tol
    assert np.max(np.abs(o[0, 1, 0] - (v1 + v2))) > 0.1
    np.testing.assert_allclose(S_T[0, 0], np.outer(key, v2), atol=1e-14)


def test_capacity_orthonormal_keys():
    """alpha = 1, beta = 1, S0 = 0: dk orthonormal keys are all recalled exactly;
    a (dk+1)-th key necessarily interferes with earlier memories."""
    rng = np.random.default_rng(6)
    dk, dv = 6, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm.T                                   # rows orthonormal
    vals = rng.standard_normal((dk, dv))
    # write all keys, then read each with beta = 0 (pure read, alpha = 1)
    T = 2 * dk
    k = np.concatenate([keys, keys])[None, :, None]
    q = k.copy()
    v = np.concatenate([vals, np.zeros((dk, dv))])[None, :, None]
    beta = np.concatenate([np.ones(dk), np.zeros(dk)])[None, :, None]
    z = np.full((1, T, 1, dk), -1e4)
    o, _ = oracle.prefill(q, k, v, z, beta, np.array([0.0]), None)
    np.testing.assert_allclose(o[0, dk:, 0], vals, atol=1e-12)
    # one more (non-orthogonal) key written after the dk: recall of key 0 breaks
    extra = rng.standard_normal(dk)
    extra /= np.linalg.norm(extra)
    k2 = np.concatenate([keys, extra[None], keys[:1]])[None, :, None]
    v2 = np.concatenate([vals, rng.standard_normal((1, dv)), np.zeros((1, dv))])[None, :, None]
    beta2 = np.concatenate([np.ones(dk + 1), np.zeros(1)])[None, :, None]
    z2 = np.full((1, dk + 2, 1, dk), -1e4)
    o2, _ = oracle.prefill(k2.copy(), k2, v2, z2, beta2, np.array([0.0]), None)
    assert np.max(np.abs(o2[0, -1, 0] - vals[0])) > 1e-3


# --------------------------------------------- brute force, chunked ----

@pytest.mark.parametrize("shape", [(1, 5, 1, 3, 2), (2, 7, 2, 4, 5), (1, 12, 1, 6, 3)])
def test_brute_force_expansion(shape):
    B, T, H, dk, dv = shape
    rng = np.random.default_rng(sum(shape))
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    ob, Sb = brute_force(q, k, v, z, beta, A, S0)
    assert relerr(o, ob) < 1e-13
    assert relerr(S_T, Sb) < 1e-13


@pytest.mark.parametrize("chunk", [1, 2, 3, 16, 32, 64, 100])
@pytest.mark.parametrize("z_mean", [0.0, 2.0, -6.0])
def test_chunked_form_agrees(chunk, z_mean):
    """The chunk-parallel algebra reproduces the sequential recurrence, for
    chunk lengths that do and do not divide T (T = 100)."""
    rng = np.random.default_rng(int(chunk * 10 + z_mean * 3 + 100))
    B, T, H, dk, dv = 1, 100, 2, 8, 6
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv, z_mean=z_mean)
    S0 = 0.5 * rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    oc, Sc = chunked(q, k, v, z, beta, A, S0, chunk=chunk)
    assert relerr(o, oc) < 1e-11
    assert relerr(S_T, Sc) < 1e-11


# ------------------------------------------------------- invariants ----

def test_split_sequence_carries_state():
    """run [0,T) == run [0,t) then [t,T) with S0 := S_t (state checkpoint at a
    token boundary)."""
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 2, 37, 3, 5, 4
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    for t in (0, 1, 16, 36, 37):
        sl1, sl2 = slice(0, t), slice(t, T)
        o1, S1 = oracle.prefill(q[:, sl1], k[:, sl1], v[:, sl1], z[:, sl1], beta[:, sl1], A, S0)
        o2, S2 = oracle.prefill(q[:, sl2], k[:, sl2], v[:, sl2], z[:, sl2], beta[:, sl2], A, S1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
        assert np.array_equal(S2, S_T)


def test_chained_oracle_helper_equals_one_run():
    """The GPU tests' full-length reference (tests/gpu_helpers.py) runs the
    oracle segment by segment over a head subset; on a small case it must give
    exactly the one-shot oracle's numbers for those heads."""
    import torch
    from tests.gpu_helpers import oracle_prefill_chained
    rng = np.random.default_rng(17)
    B, T, H, dk, dv = 1, 45, 4, 6, 6
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    # fp32 inputs, as the GPU tests hand over (the helper reads tensors as fp32)
    q, k, v, z, beta, A, S0 = (x.astype(np.float32) for x in (q, k, v, z, beta, A, S0))
    inp = {n: torch.from_numpy(x) for n, x in
           dict(q=q, k=k, v=v, z=z, beta=beta, A=A, S0=S0).items()}
    heads = [1, 3]
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    oc, Sc = oracle_prefill_chained(inp, heads, seg=8)
    assert np.array_equal(oc, o[:, :, heads].astype(np.float32))
    assert np.array_equal(Sc, S_T[:, heads])


def test_linearity_and_independence():
    rng = np.random.default_rng(8)
    B, T, H, dk, dv = 2, 20, 4, 5, 3
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv)
    v2 = rng.standard_normal(v.shape)
    S0a, S0b = rng.standard_normal((2, B, H, dk, dv))
    oa, Sa = oracle.prefill(q, k, v, z, beta, A, S0a)
    ob, Sb = oracle.prefill(q, k, v2, z, beta, A, S0b)
    os_, Ss = oracle.prefill(q, k, 2.0 * v - 3.0 * v2, z, beta, A, 2.0 * S0a - 3.0 * S0b)
    assert relerr(os_, 2 * oa - 3 * ob) < 1e-12
    assert relerr(Ss, 2 * Sa - 3 * Sb) < 1e-12
    # heads are independent: permuting heads (and A) permutes the outputs
    perm = np.array([2, 0, 3, 1])
    op, Sp = oracle.prefill(q[:, :, perm], k[:, :, perm], v[:, :, perm], z[:, :, perm],
                            beta[:, :, perm], A[perm], S0a[:, perm])
    assert np.array_equal(op, oa[:, :, perm]) and np.array_equal(Sp, Sa[:, perm])
    # value columns evolve independently
    oc, Sc = oracle.prefill(q, k, v[..., :1], z, beta, A, S0a[..., :1])
    assert np.array_equal(oc, oa[..., :1]) and np.array_equal(Sc, Sa[..., :1])


def test_non_expansive_step():
    """||k|| <= 1, beta in [0,1]: ||S_t||_F <= ||S_{t-1}||_F + beta ||k|| ||v||."""
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 1, 60, 2, 7, 5
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv, z_mean=-3.0)
    S = rng.standard_normal((B, H, dk, dv))
    for t in range(T):
        _, Sn = oracle.prefill(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], z[:, t:t + 1],
                               beta[:, t:t + 1], A, S)
        for h in range(H):
            lhs = np.linalg.norm(Sn[0, h])
            rhs = np.linalg.norm(S[0, h]) + beta[0, t, h] * np.linalg.norm(k[0, t, h]) * \
                np.linalg.norm(v[0, t, h])
            assert lhs <= rhs * (1 + 1e-14)
        S = Sn


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(10)
    B, T, H, dk, dv = 3, 11, 2, 4, 6
    q, k, v, z, beta, A = _rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    S = S0
    for t in range(T):
        ot, S = oracle.decode_step(q[:, t], k[:, t], v[:, t], z[:, t], beta[:, t], A, S)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(S, S_T)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(11)
    q, k, v, z, beta, A = _rand_inputs(rng, 2, 0, 3, 4, 5)
    S0 = rng.standard_normal((2, 3, 4, 5))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0)
    assert o.shape == (2, 0, 3, 5)
    assert np.array_equal(S_T, S0)
    _, S_T0 = oracle.prefill(q, k, v, z, beta, A, None)
    assert np.all(S_T0 == 0.0)


def test_thread_count_does_not_change_result():
    rng = np.random.default_rng(12)
    q, k, v, z, beta, A = _rand_inputs(rng, 2, 33, 5, 6, 4)
    r1 = oracle.prefill(q, k, v, z, beta, A, None, threads=1)
    r8 = oracle.prefill(q, k, v, z, beta, A, None, threads=8)
    assert np.array_equal(r1[0], r8[0]) and np.array_equal(r1[1], r8[1])


def test_log_decay_cumsum_window_bound():
    """Every 16-token window of the log-decay stays >= -80 (range claim)."""
    rng = np.random.default_rng(13)
    z = rng.standard_normal((4096, 8)) + 2.0
    g = np.stack([oracle.gate(z[:, j], a) for j, a in enumerate(np.linspace(-1, 1, 8))], 1)
    np.testing.assert_allclose(g, np.stack([log_decay(z[:, j], a) for j, a in
                                            enumerate(np.linspace(-1, 1, 8))], 1), rtol=1e-14)
    win = np.lib.stride_tricks.sliding_window_view(g, 16, axis=0).sum(-1)
    assert win.min() >= -80.0
