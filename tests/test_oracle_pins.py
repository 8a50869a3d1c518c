"""The fp64 oracle against what the pages and mathematics fix (CPU only).

Each pin in tests/oracle_pins.py runs against the oracle, and the mutation test
plants plausible mistakes in copies of the oracle source and checks that every
mutant fails at least one pin.
"""
import functools
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    for label, err, tol in pin(oracle.fwd, oracle.decode):
        assert err <= tol, f"{label}: {err:.3e} > {tol:.1e}"


# Plausible mistakes, each a single textual change of gdr2_oracle.c.
MUTANTS = {
    "no decay": ("S[i * dv + j] *= alpha;", "S[i * dv + j] *= 1.0 + 0.0 * alpha;"),
    "linearised decay": ("const double alpha = exp(g[i]);", "const double alpha = 1.0 + g[i];"),
    "erase gate dropped": ("const double e = b[i] * k[i];", "const double e = k[i];"),
    "erase reads b only": ("const double e = b[i] * k[i];", "const double e = b[i];"),
    "write gate dropped": ("k[i] * (w[j] * v[j] - r[j])", "k[i] * (v[j] - r[j])"),
    "residual sign": ("k[i] * (w[j] * v[j] - r[j])", "k[i] * (w[j] * v[j] + r[j])"),
    "gated write direction": ("S[i * dv + j] += k[i] * (", "S[i * dv + j] += b[i] * k[i] * ("),
    "output reads with k": ("o[j] += S[i * dv + j] * q[i];", "o[j] += S[i * dv + j] * k[i];"),
    "output from the pre-edit state": ("o[j] += S[i * dv + j] * q[i];",
                                       "o[j] += (S[i * dv + j] - k[i] * (w[j] * v[j] - r[j])) * q[i];"),
    "read before decay": ("r[j] += S[i * dv + j] * e;", "r[j] += S[i * dv + j] * e / exp(g[i]);"),
    "no state reset": ("if (S0) memcpy(S, S0 + (size_t)nh * sz, sizeof(double) * sz);",
                       "if (S0) memcpy(S, S0 + (size_t)h * sz, sizeof(double) * sz);"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdr2_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    path_c = os.path.join(mutant_dir, name.replace(" ", "_") + ".c")
    path_so = path_c[:-2] + ".so"
    open(path_c, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o",
                           path_so, path_c, "-lm"])
    lib = oracle.load_library(path_so)
    fwd = functools.partial(oracle.fwd, lib=lib)
    dec = functools.partial(oracle.decode, lib=lib)
    failed = []
    for pin in P.ALL_PINS:
        for label, err, tol in pin(fwd, dec):
            if not (err <= tol):
                failed.append(label)
    assert failed, f"mutant {name!r} passed every pin"


def test_oracle_threads_report():
    assert oracle.max_threads() >= 1


def test_masked_pairs_left_untouched():
    q, k, v, g, b, w = P.rand_inputs(30, 2, 10, 3, 4, 4)
    mask = np.zeros((2, 3), bool)
    mask[1, 2] = True
    o, ST = oracle.fwd(q, k, v, g, b, w, mask=mask)
    of, STf = oracle.fwd(q, k, v, g, b, w)
    assert np.array_equal(o[1, :, 2], of[1, :, 2]) and np.array_equal(ST[1, 2], STf[1, 2])
    assert not o[0].any() and not ST[0].any() and not o[1, :, :2].any()
