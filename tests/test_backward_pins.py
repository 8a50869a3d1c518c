"""The fp64 backward oracle against the facts pinned in tests/backward_pins.py
(CPU only), and plausible mistakes planted in copies of its C source, each of
which must fail at least one pin."""
import functools
import os
import subprocess

import pytest

import oracle
from tests import backward_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    for label, err, tol in pin(oracle.bwd):
        assert err <= tol, f"{label}: {err:.3e} > {tol:.1e}"


MUTANTS = {
    "dq from the pre-edit state": ("acc += Sn[i * dv + j] * dout[j];", "acc += Sb[i * dv + j] * dout[j];"),
    "decay gradient without alpha": ("dg[i] = da * a;", "dg[i] = da;"),
    "read gradient sign": ("dr[j] = -dr[j];                          /* dL/dr */", "dr[j] = dr[j];"),
    "erase gradient misses k": ("db[i] = de * k[i];", "db[i] = de;"),
    "state gradient not decayed": ("dS[i * dv + j] *= a;", "dS[i * dv + j] *= 1.0;"),
    "key gradient misses the erase path": ("dk_[i] += de * b[i];", "dk_[i] += 0.0 * de * b[i];"),
    "write gradient uses w": ("dw[j] = dr[j] * v[j];", "dw[j] = dr[j] * w[j];"),
    "initial-state gradient of the wrong pair": ("if (dS0) memcpy(dS0 + (size_t)nh * sz", "if (dS0) memcpy(dS0 + (size_t)h * sz"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_bwd_mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdr2_oracle_bwd.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    path_c = os.path.join(mutant_dir, name.replace(" ", "_") + ".c")
    path_so = path_c[:-2] + ".so"
    open(path_c, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o",
                           path_so, path_c, "-lm"])
    bwd = functools.partial(oracle.bwd, lib=oracle.load_bwd_library(path_so))
    failed = []
    for pin in P.ALL_PINS:
        for label, err, tol in pin(bwd):
            if not (err <= tol):
                failed.append(label)
    assert failed, f"mutant {name!r} passed every pin"
