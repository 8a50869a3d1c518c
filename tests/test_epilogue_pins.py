"""The output-epilogue oracle against the facts pinned in
tests/epilogue_pins.py (CPU only), and plausible mistakes planted in copies of
the oracle's source, each of which must fail at least one pin."""
import importlib.util
import os

import pytest

from oracle import epilogue
from tests import epilogue_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    for label, err, tol in pin(epilogue.norm_gate, epilogue.silu):
        assert err <= tol, f"{label}: {err:.3e} > {tol:.1e}"


MUTANTS = {
    "sum instead of mean": ("np.mean(g * g, axis=-1, keepdims=True)", "np.sum(g * g, axis=-1, keepdims=True)"),
    "eps outside the root": ("np.sqrt(mean_sq + float(eps))", "(np.sqrt(mean_sq) + float(eps))"),
    "no square root": ("np.sqrt(mean_sq + float(eps))", "(mean_sq + float(eps))"),
    "sigmoid gate": ("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))"),
    "gate sign": ("return z / (1.0 + np.exp(-z))", "return z / (1.0 + np.exp(z))"),
    "weight dropped": ("y = y * w", "y = y * 1.0"),
    "weight reversed": ("y = y * w", "y = y * w[::-1]"),
    "whole-width norm": ("g = o.reshape(-1, d // group, group)", "g = o.reshape(-1, 1, d)"),
    "gate reads o": ("return y * silu(z)", "return y * silu(o)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(epilogue.__file__).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    path = os.path.join(tmp_path, "epilogue_mutant.py")
    open(path, "w").write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("epilogue_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in P.ALL_PINS:
        try:
            res = pin(mod.norm_gate, mod.silu)
        except Exception as exc:  # a mutant that breaks a shape check is caught too
            failed.append(f"{pin.__name__}: {exc!r}")
            continue
        failed += [label for label, err, tol in res if not (err <= tol)]
    assert failed, f"mutant {name!r} passed every pin"
