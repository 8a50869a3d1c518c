"""The gate-prologue oracle against the facts pinned in tests/prologue_pins.py
(CPU only), and plausible mistakes planted in copies of the oracle's source,
each of which must fail at least one pin."""
import importlib.util
import os

import pytest

from oracle import prologue
from tests import prologue_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    for label, err, tol in pin(prologue):
        assert err <= tol, f"{label}: {err:.3e} > {tol:.1e}"


MUTANTS = {
    "decay magnitude not exponentiated": ("return -np.exp(a) * softplus(f + delta)",
                                          "return -a * softplus(f + delta)"),
    "decay sign": ("return -np.exp(a) * softplus(f + delta)", "return np.exp(a) * softplus(f + delta)"),
    "decay bias dropped": ("return -np.exp(a) * softplus(f + delta)", "return -np.exp(a) * softplus(f)"),
    "decay bias subtracted": ("return -np.exp(a) * softplus(f + delta)",
                              "return -np.exp(a) * softplus(f - delta)"),
    "erase scale ignored": ("b = b_scale * sigmoid(b)", "b = sigmoid(b)"),
    "write gate as SiLU": ("w = sigmoid(w)", "w = w * sigmoid(w)"),
    "L2 eps outside the root": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))",
                                "x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + float(eps))"),
    "no L2 root": ("x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))",
                   "x / (np.sum(x * x, axis=-1, keepdims=True) + float(eps))"),
    "tiled value heads": ("return np.repeat(_f64(x), int(group), axis=-2)",
                          "return np.concatenate([_f64(x)] * int(group), axis=-2)"),
    "softplus as exp": ("return np.logaddexp(0.0, _f64(x))", "return np.exp(_f64(x))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(prologue.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    path = os.path.join(tmp_path, "prologue_mutant.py")
    open(path, "w").write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("prologue_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in P.ALL_PINS:
        try:
            res = pin(mod)
        except Exception as exc:
            failed.append(f"{pin.__name__}: {exc!r}")
            continue
        failed += [label for label, err, tol in res if not (err <= tol)]
    assert failed, f"mutant {name!r} passed every pin"
