"""Pins for the prologue oracle (CPU only): short causal depthwise convolution,
SiLU and q/k L2 normalization, and their composition with the recurrence.

The readings these check (tap W-1 weighs the current token, the state holds the
last W-1 raw inputs oldest first, x / sqrt(sum x^2 + eps)) are stated in
``oracle/prologue.py``.  Every check reaches the expected value by a route other
than the oracle's own: numpy.convolve, explicit delays, closed forms, scipy's
logistic function, or invariants that a dropped or misplaced term breaks.  The
mutant test at the end plants one mistake at a time in a copy of the module and
requires the battery to fail on each.
"""
import importlib.util
import math
import os
import sys

import numpy as np
import pytest

import oracle
from oracle import prologue
from tests.kda_pins import relerr

SRC = os.path.join(os.path.dirname(oracle.__file__), "prologue.py")


def _rand(rng, B, T, H, d, W):
    x = rng.standard_normal((B, T, H, d))
    w = rng.standard_normal((H, d, W))
    st = rng.standard_normal((B, W - 1, H, d))
    return x, w, st


# ------------------------------------------------------- the pin battery ----
# Each check takes the module under test and returns True when it holds.

def pin_numpy_convolve(mod):
    """Each channel equals numpy's full convolution of state + input with the
    reversed taps (numpy.convolve flips its second argument); with act="silu"
    each output is then r / (1 + e^-r)."""
    rng = np.random.default_rng(3)
    for W in (1, 2, 3, 4):
        x, w, st = _rand(rng, 2, 11, 2, 3, W)
        y, _ = mod.short_conv(x, w, st)
        ys, _ = mod.short_conv(x, w, st, act="silu")
        for b in range(2):
            for h in range(2):
                for c in range(3):
                    seq = np.concatenate([st[b, :, h, c], x[b, :, h, c]])
                    ref = np.convolve(seq, w[h, c, ::-1], mode="valid")
                    if np.max(np.abs(y[b, :, h, c] - ref)) > 1e-13:
                        return False
                    refs = np.array([r / (1.0 + math.exp(-r)) for r in ref])
                    if np.max(np.abs(ys[b, :, h, c] - refs)) > 1e-13:
                        return False
    return True


def pin_delta_taps(mod):
    """A unit tap on the current token is the identity; a unit tap on the
    oldest one delays by W-1 tokens, reading the state first."""
    rng = np.random.default_rng(4)
    W = 4
    x, _, st = _rand(rng, 1, 9, 2, 3, W)
    w_id = np.zeros((2, 3, W)); w_id[..., W - 1] = 1.0
    w_old = np.zeros((2, 3, W)); w_old[..., 0] = 1.0
    y_id, _ = mod.short_conv(x, w_id, st)
    y_old, _ = mod.short_conv(x, w_old, st)
    delayed = np.concatenate([st, x[:, :9 - (W - 1)]], axis=1)
    return np.array_equal(y_id, x) and np.array_equal(y_old, delayed)


def pin_state_contents(mod):
    """The new state holds the last W-1 raw inputs, oldest first, also when the
    segment is shorter than W-1 (then part of the old state shifts down)."""
    rng = np.random.default_rng(5)
    W = 4
    x, w, st = _rand(rng, 1, 7, 1, 2, W)
    _, ns = mod.short_conv(x, w, st)
    if not np.array_equal(ns, x[:, 4:7]):
        return False
    _, ns1 = mod.short_conv(x[:, :1], w, st)
    if not np.array_equal(ns1, np.concatenate([st[:, 1:], x[:, :1]], axis=1)):
        return False
    _, ns0 = mod.short_conv(x[:, :0], w, st)   # an empty segment keeps the state
    return np.array_equal(ns0, st)


def pin_split_segment(mod):
    """Convolving T tokens at once equals two segments with the state carried."""
    rng = np.random.default_rng(6)
    for W in (2, 4):
        x, w, st = _rand(rng, 2, 13, 2, 3, W)
        y, ns = mod.short_conv(x, w, st, act="silu")
        for cut in (0, 1, 2, 7, 13):
            y1, s1 = mod.short_conv(x[:, :cut], w, st, act="silu")
            y2, s2 = mod.short_conv(x[:, cut:], w, s1, act="silu")
            if relerr(np.concatenate([y1, y2], axis=1), y) > 1e-15 or not np.array_equal(s2, ns):
                return False
    return True


def pin_linearity(mod):
    rng = np.random.default_rng(7)
    x1, w1, _ = _rand(rng, 1, 8, 2, 4, 3)
    x2, w2, _ = _rand(rng, 1, 8, 2, 4, 3)
    a, b = 0.75, -1.25
    y12, _ = mod.short_conv(a * x1 + b * x2, w1)
    y1, _ = mod.short_conv(x1, w1)
    y2, _ = mod.short_conv(x2, w1)
    yw, _ = mod.short_conv(x1, a * w1 + b * w2)
    yw2, _ = mod.short_conv(x1, w2)
    return relerr(y12, a * y1 + b * y2) < 1e-14 and relerr(yw, a * y1 + b * yw2) < 1e-14


def pin_silu(mod):
    xs = np.array([-30.0, -2.5, -0.1, 0.0, 0.3, 1.0, 4.0, 30.0])
    ref = np.array([x / (1.0 + math.exp(-x)) for x in xs])
    y = mod.silu(xs)
    return y[3] == 0.0 and np.max(np.abs(y - ref)) < 1e-14


def pin_l2norm(mod):
    if not np.allclose(mod.l2norm(np.array([3.0, 4.0]), 0.0), [0.6, 0.8], rtol=0, atol=1e-16):
        return False
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 7, 16))
    n = mod.l2norm(x, 0.0)
    if np.max(np.abs(np.linalg.norm(n, axis=-1) - 1.0)) > 1e-14:
        return False
    if relerr(mod.l2norm(3.5 * x, 0.0), n) > 1e-15:
        return False
    # the guard: sum x^2 + eps under the root, closed form for one channel
    eps = 0.25
    s = mod.l2norm(np.array([[1.5]]), eps)[0, 0]
    if abs(s - 1.5 / math.sqrt(1.5 * 1.5 + eps)) > 1e-15:
        return False
    return np.array_equal(mod.l2norm(np.zeros((2, 4)), 1e-6), np.zeros((2, 4)))


def pin_conv_norm(mod):
    """q and k come out with unit norm (up to eps), v is the bare convolution,
    and with identity taps the prologue only normalizes."""
    rng = np.random.default_rng(9)
    W = 3
    q, wq, sq = _rand(rng, 1, 6, 2, 8, W)
    k, wk, sk = _rand(rng, 1, 6, 2, 8, W)
    v, wv, sv = _rand(rng, 1, 6, 2, 5, W)
    qh, kh, vc, (nq, nk, nv) = mod.conv_norm(q, k, v, wq, wk, wv, sq, sk, sv, "silu", 0.0)
    if np.max(np.abs(np.linalg.norm(qh, axis=-1) - 1)) > 1e-14:
        return False
    if np.max(np.abs(np.linalg.norm(kh, axis=-1) - 1)) > 1e-14:
        return False
    v_ref, _ = mod.short_conv(v, wv, sv, "silu")
    if not np.array_equal(vc, v_ref) or not np.array_equal(nv, v[:, 6 - (W - 1):]):
        return False
    wid = np.zeros((2, 8, W)); wid[..., W - 1] = 1.0
    widv = np.zeros((2, 5, W)); widv[..., W - 1] = 1.0
    qh, kh, vc, _ = mod.conv_norm(q, k, v, wid, wid, widv, act="none", eps=0.0)
    return (relerr(qh, q / np.linalg.norm(q, axis=-1, keepdims=True)) < 1e-15
            and relerr(kh, k / np.linalg.norm(k, axis=-1, keepdims=True)) < 1e-15
            and np.array_equal(vc, v))


BATTERY = [pin_numpy_convolve, pin_delta_taps, pin_state_contents, pin_split_segment,
           pin_linearity, pin_silu, pin_l2norm, pin_conv_norm]


@pytest.mark.parametrize("pin", BATTERY, ids=lambda f: f.__name__)
def test_prologue_pin(pin):
    assert pin(prologue)


# ------------------------------------------------- composed with the path ----

def _layer_inputs(rng, B, T, H, dk, dv, W):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk))
    beta = rng.uniform(0, 1, (B, T, H))
    A = rng.uniform(-1, 1, H)
    wq = rng.standard_normal((H, dk, W)) * 0.5
    wk = rng.standard_normal((H, dk, W)) * 0.5
    wv = rng.standard_normal((H, dv, W)) * 0.5
    st = (rng.standard_normal((B, W - 1, H, dk)), rng.standard_normal((B, W - 1, H, dk)),
          rng.standard_normal((B, W - 1, H, dv)))
    S0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, z, beta, A, wq, wk, wv, st, S0


def test_prefill_conv_identity_taps_is_prefill():
    """Identity taps, pre-normalized q, k and eps = 0: the prologue is a no-op
    and the composed oracle is the pinned recurrence."""
    rng = np.random.default_rng(10)
    B, T, H, dk, dv, W = 1, 9, 2, 6, 5, 4
    q, k, v, z, beta, A, _, _, _, st, S0 = _layer_inputs(rng, B, T, H, dk, dv, W)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    wid = np.zeros((H, dk, W)); wid[..., W - 1] = 1.0
    widv = np.zeros((H, dv, W)); widv[..., W - 1] = 1.0
    o, S_T, _ = oracle.prefill_conv(q, k, v, z, beta, A, wid, wid, widv, st, "none", 0.0, S0)
    o_ref, S_ref = oracle.prefill(q, k, v, z, beta, A, S0)
    assert relerr(o, o_ref) < 1e-14 and relerr(S_T, S_ref) < 1e-14


@pytest.mark.parametrize("act", ["none", "silu"])
def test_decode_steps_equal_one_prefill(act):
    """T decode steps, carrying both states, equal one prefill of the T tokens."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv, W = 2, 7, 2, 6, 5, 4
    q, k, v, z, beta, A, wq, wk, wv, st, S0 = _layer_inputs(rng, B, T, H, dk, dv, W)
    o, S_T, cs = oracle.prefill_conv(q, k, v, z, beta, A, wq, wk, wv, st, act, 1e-6, S0)
    S, state = S0, st
    for t in range(T):
        ot, S, state = oracle.decode_step_conv(q[:, t], k[:, t], v[:, t], z[:, t], beta[:, t],
                                               A, wq, wk, wv, state, S, act, 1e-6)
        assert relerr(ot, o[:, t]) < 1e-12
    assert relerr(S, S_T) < 1e-12
    for a, b in zip(state, cs):
        assert np.array_equal(a, b)


# --------------------------------------------------------------- mutants ----

MUTANTS = {
    "taps_reversed": ("w[None, None, :, :, j] * xp[:, j:j + T]",
                      "w[None, None, :, :, W - 1 - j] * xp[:, j:j + T]"),
    "window_off_by_one": ("xp[:, j:j + T]", "xp[:, j + 1:j + 1 + T] if j + 1 + T <= xp.shape[1] "
                                            "else xp[:, j:j + T]"),
    "state_newest_first": ("new_state = xp[:, xp.shape[1] - (W - 1):]",
                           "new_state = xp[:, xp.shape[1] - (W - 1):][:, ::-1]"),
    "state_from_outputs": ("new_state = xp[:, xp.shape[1] - (W - 1):]",
                           "new_state = np.concatenate([state, y], axis=1)[:, T:]"),
    "eps_outside_root": ("np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)",
                         "(np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + eps)"),
    "norm_over_heads": ("np.sum(x * x, axis=-1, keepdims=True)",
                        "np.sum(x * x, axis=-2, keepdims=True)"),
    "silu_sign": ("return x * expit(x)", "return x * expit(-x)"),
    "v_normalized": ("return l2norm(qc, eps), l2norm(kc, eps), vc, (sq, sk, sv)",
                     "return l2norm(qc, eps), l2norm(kc, eps), l2norm(vc, eps), (sq, sk, sv)"),
    "silu_dropped": ("    if act == \"silu\":\n        y = silu(y)",
                     "    if act == \"silu\":\n        y = y"),
}


def _load_mutant(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = tmp_path / f"prologue_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"_prologue_mutant_{name}", str(path))
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prologue_mutant_is_caught(tmp_path, name):
    mod = _load_mutant(tmp_path, name)

    def holds(pin):
        try:
            with np.errstate(all="ignore"):
                return bool(pin(mod))
        except Exception:   # a mutant that cannot even run fails the pin
            return False

    failed = [p.__name__ for p in BATTERY if not holds(p)]
    assert failed, f"mutant {name} passed every pin"
