"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pins catch every one of them.

Each mutant is a one-line edit of ``oracle/kda_oracle.c`` compiled into a
temporary directory; the shipped oracle is never touched.  The battery below
re-runs the independent checks of ``test_oracle_pins.py`` (brute force,
closed forms, overwrite, gate values) against the mutant; at least one must
fail for each edit.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests.kda_pins import brute_force, decay, relerr

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "drop_erase": ("S[i * dv + j] -= bt * kt[i] * w[j];", "(void)w;"),
    "erase_sign": ("S[i * dv + j] -= bt * kt[i] * w[j];", "S[i * dv + j] += bt * kt[i] * w[j];"),
    "decay_on_value_columns": ("S[i * dv + j] *= alpha[i];", "S[i * dv + j] *= alpha[j % dk];"),
    "gate_sign": ("exp(-(c * z))", "exp(c * z)"),
    "gate_scale_not_exponentiated": ("const double c = exp(A[h]);", "const double c = A[h];"),
    "read_before_update": ("ot[j] += S[i * dv + j] * qt[i];",
                           "ot[j] += (S[i * dv + j] - bt * kt[i] * (vt[j] - w[j])) * qt[i];"),
    "write_without_beta": ("S[i * dv + j] += bt * kt[i] * vt[j];", "S[i * dv + j] += kt[i] * vt[j];"),
    "wrong_g_min": ("#define KDA_ORACLE_GMIN (-5.0)", "#define KDA_ORACLE_GMIN (-4.0)"),
    "erase_with_unfaded_state": ("w[j] += kt[i] * S[i * dv + j];",
                                 "w[j] += kt[i] * S[i * dv + j] / alpha[i];"),
    "read_with_key": ("ot[j] += S[i * dv + j] * qt[i];", "ot[j] += S[i * dv + j] * kt[i];"),
}


def _build_mutant(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path_c = tmp_path / f"{name}.c"
    path_c.write_text(src.replace(old, new))
    path_so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                    str(path_so), str(path_c), "-lm"], check=True)
    return oracle.load_variant(str(path_so))


def _battery(lib):
    """Return the names of the pins the given oracle build fails."""
    failed = []
    rng = np.random.default_rng(42)
    B, T, H, dk, dv = 1, 6, 2, 4, 3
    q = rng.standard_normal((B, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk))
    beta = rng.uniform(0, 1, (B, T, H))
    A = rng.uniform(-1, 1, H)
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.prefill(q, k, v, z, beta, A, S0, lib=lib)
    ob, Sb = brute_force(q, k, v, z, beta, A, S0)
    if relerr(o, ob) > 1e-12 or relerr(S_T, Sb) > 1e-12:
        failed.append("brute_force")
    # beta = 0 closed form
    o0, S0T = oracle.prefill(q, k, v, z, 0 * beta, A, S0, lib=lib)
    cum = np.ones((H, dk))
    exp_o = np.zeros_like(o0)
    for t in range(T):
        cum = cum * np.stack([decay(z[0, t, h], A[h]) for h in range(H)])
        exp_o[0, t] = np.einsum("hdv,hd->hv", S0[0], cum * q[0, t])
    if relerr(o0, exp_o) > 1e-12 or relerr(S0T[0], cum[..., None] * S0[0]) > 1e-12:
        failed.append("beta_zero")
    # overwrite
    key = np.eye(dk)[0]
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    ow, _ = oracle.prefill(np.stack([key, key])[None, :, None], np.stack([key, key])[None, :, None],
                           np.stack([v1, v2])[None, :, None], np.full((1, 2, 1, dk), -1e4),
                           np.ones((1, 2, 1)), np.array([0.3]), None, lib=lib)
    if np.max(np.abs(ow[0, 1, 0] - v2)) > 1e-14:
        failed.append("overwrite")
    g = oracle.gate(np.array([0.0, 1e4, -1e4, 1.0]), 0.5, lib=lib)
    if not (g[0] == -2.5 and g[1] == -5.0 and g[2] == 0.0
            and abs(g[3] + 5.0 / (1.0 + np.exp(-np.exp(0.5)))) < 1e-14):
        failed.append("gate_values")
    return failed


def test_shipped_oracle_passes_battery():
    assert _battery(None) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    lib = _build_mutant(tmp_path, name)
    assert _battery(lib), f"mutant {name} passed every pin"
