"""Pins for the reverse-mode oracle (CPU only).

``oracle.prefill_bwd`` is the adjoint of the sequential recurrence, written
step by step.  It is pinned against central finite differences of the forward
oracle (itself pinned in test_oracle_pins.py) on every input element of small
cases with dk != dv, against the T = 0 identity, and a battery of planted
mistakes in copies of its C source must each fail the finite-difference pin.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.kda_pins import chunked_bwd, relerr

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


def _case(seed, B=2, T=5, H=2, dk=3, dv=4, beta_zero=False):
    rng = np.random.default_rng(seed)
    x = {
        "q": rng.standard_normal((B, T, H, dk)) * 0.7,
        "k": rng.standard_normal((B, T, H, dk)) * 0.5,
        "v": rng.standard_normal((B, T, H, dv)),
        "z": rng.standard_normal((B, T, H, dk)),
        "beta": np.zeros((B, T, H)) if beta_zero else rng.uniform(0.1, 0.9, (B, T, H)),
        "A": rng.uniform(-1, 1, (H,)),
        "S0": rng.standard_normal((B, H, dk, dv)) * 0.5,
    }
    G = rng.standard_normal((B, T, H, dv))        # dL/do
    Hs = rng.standard_normal((B, H, dk, dv))      # dL/dS_T
    return x, G, Hs


def _loss(x, G, Hs):
    o, S_T = oracle.prefill(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["S0"],
                            threads=1)
    return float(np.sum(o * G) + np.sum(S_T * Hs))


NAMES = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("z", "dz"), ("beta", "dbeta"), ("A", "dA"),
         ("S0", "dS0")]


def finite_difference_errors(grads, x, G, Hs, h=1e-6):
    """Largest |adjoint - central difference| / max(1, max|grad|) per input."""
    errs = {}
    for name, gname in NAMES:
        base = x[name]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = dict(x); xp[name] = base.copy(); xp[name][idx] += h
            xm = dict(x); xm[name] = base.copy(); xm[name][idx] -= h
            fd[idx] = (_loss(xp, G, Hs) - _loss(xm, G, Hs)) / (2 * h)
        g = grads[gname]
        errs[name] = float(np.max(np.abs(g - fd)) / max(1.0, np.max(np.abs(fd))))
    return errs


def _grads(x, G, Hs, lib=None):
    return oracle.prefill_bwd(x["q"], x["k"], x["v"], x["z"], x["beta"], x["A"], x["S0"], G,
                              Hs, threads=1, lib=lib)


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed):
    x, G, Hs = _case(seed)
    errs = finite_difference_errors(_grads(x, G, Hs), x, G, Hs)
    assert max(errs.values()) < 1e-7, errs


def test_backward_long_memory_and_unit_keys():
    """Decays near 1 (z ~ N(-6,1)), unit keys, beta up to 1: the erase terms
    dominate and the state carries across all tokens."""
    x, G, Hs = _case(3, B=1, T=7, H=1, dk=4, dv=3)
    x["z"] = x["z"] - 6.0
    x["k"] = x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)
    x["beta"] = np.clip(x["beta"] + 0.3, 0, 1)
    errs = finite_difference_errors(_grads(x, G, Hs), x, G, Hs)
    assert max(errs.values()) < 1e-7, errs


def test_backward_beta_zero():
    """With beta = 0 the values never enter: dv = 0 exactly."""
    x, G, Hs = _case(4, beta_zero=True)
    g = _grads(x, G, Hs)
    assert np.array_equal(g["dv"], np.zeros_like(g["dv"]))
    errs = finite_difference_errors(g, x, G, Hs)
    assert max(errs.values()) < 1e-7, errs


def test_backward_empty_sequence():
    """T = 0: S_T = S0, so dS0 = dL/dS_T and dA = 0."""
    x, G, Hs = _case(5, T=0)
    g = _grads(x, G, Hs)
    assert np.array_equal(g["dS0"], Hs)
    assert np.array_equal(g["dA"], np.zeros_like(g["dA"]))


def test_backward_thread_count_invariant():
    x, G, Hs = _case(6, B=3, T=9, H=4, dk=5, dv=3)
    g1 = oracle.prefill_bwd(*(x[n] for n in ("q", "k", "v", "z", "beta", "A", "S0")), G, Hs,
                            threads=1)
    g8 = oracle.prefill_bwd(*(x[n] for n in ("q", "k", "v", "z", "beta", "A", "S0")), G, Hs,
                            threads=8)
    for key in g1:
        assert np.array_equal(g1[key], g8[key]), key


MUTANTS = {
    "erase_beta_sign": ("dbt -= kt[i] * sw;", "dbt += kt[i] * sw;"),
    "fade_on_columns": ("dS[i * dv + j] = alpha[i] * dS[i * dv + j];",
                        "dS[i * dv + j] = alpha[j % dk] * dS[i * dv + j];"),
    "drop_key_through_w": ("dkt[i] += fd;", "(void)fd;"),
    "gate_without_scale": ("dzt[i] = ce * dx;", "dzt[i] = dx;"),
    "dA_without_z": ("dA_acc += ce * zt[i] * dx;", "dA_acc += ce * dx;"),
    "read_old_state": ("acc += St[i * dv + j] * dot[j];", "acc += Sp[i * dv + j] * dot[j];"),
    "dv_without_beta": ("dvt[j] = bt * sk;", "dvt[j] = sk;"),
    "sigmoid_slope": ("dg * KDA_ORACLE_GMIN * s * (1.0 - s)", "dg * KDA_ORACLE_GMIN * s"),
    "state_grad_skips_query": ("dS[i * dv + j] += qt[i] * dot[j];", "(void)qt;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    c = tmp_path / f"{name}.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(c), "-lm"], check=True)
    lib = oracle.load_variant(str(so))
    x, G, Hs = _case(0)
    errs = finite_difference_errors(_grads(x, G, Hs, lib=lib), x, G, Hs)
    assert max(errs.values()) > 1e-4, f"mutant {name} passed the finite-difference pin"


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 16])
def test_chunked_backward_model_matches_adjoint(chunk):
    """The chunk-parallel reverse mode (a model of a chunked GPU backward)
    equals the step-by-step adjoint, for chunk lengths that divide T, do not,
    and exceed it; decays near 1 included."""
    for T, zshift in ((7, 0.0), (11, -6.0), (4, 0.0)):
        x, G, Hs = _case(7 + T, B=2, T=T, H=2, dk=4, dv=3)
        x["z"] = x["z"] + zshift
        ref = _grads(x, G, Hs)
        got = chunked_bwd(*(x[n] for n in ("q", "k", "v", "z", "beta", "A", "S0")), G, Hs,
                          chunk=chunk)
        for key in ref:
            assert relerr(got[key], ref[key]) < 1e-10, (chunk, T, key)
