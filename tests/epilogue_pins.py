"""Pins for the output-epilogue oracle (RMSNorm, then a SiLU output gate).

Each pin is ``pin_x(norm_gate, silu) -> list[(label, err, tol)]`` so that the
checks run against the oracle (tests/test_epilogue_pins.py) and against
deliberately broken copies of it, each of which must fail at least one pin.
The facts pinned come from the pages' description of the block output
(Gated DeltaNet-2 pages, "Big-Picture Architecture" item 6) and from the
definitions of RMSNorm and SiLU, not from the oracle's code.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


def pin_golden(norm_gate, silu):
    """The hand-worked two-channel example (exact up to rounding)."""
    with open(os.path.join(GOLDEN, "epilogue_hand_worked_d2.json")) as f:
        gd = json.load(f)
    ln3 = math.log(3.0)
    y = norm_gate(np.array(gd["o"]), np.array(gd["z_over_ln3"]) * ln3,
                  weight=np.array(gd["weight"]), eps=gd["eps"])
    return [("golden y", rel(y, np.array(gd["expected_y_over_ln3"]) * ln3), 1e-15)]


def pin_silu(norm_gate, silu):
    """silu(z) = z * sigmoid(z): silu(0) = 0, silu(-z) = silu(z) - z,
    silu(ln 3) = (3/4) ln 3, silu -> z for large z and -> 0 for very negative z."""
    z = np.random.default_rng(1).standard_normal(64) * 4
    ln3 = math.log(3.0)
    out = [("silu(0)", abs(float(silu(np.array([0.0]))[0])), 0.0),
           ("silu(-z) = silu(z) - z", rel(silu(-z), silu(z) - z), 1e-14),
           ("silu(ln 3)", rel(silu(np.array([ln3])), [0.75 * ln3]), 1e-15),
           ("silu(40) ~ 40", rel(silu(np.array([40.0])), [40.0]), 1e-15)]
    neg = silu(np.array([-800.0]))
    out.append(("silu(-800) is 0, not NaN", float(abs(neg[0])) if np.isfinite(neg[0]) else math.inf, 0.0))
    return out


def pin_groups(norm_gate, silu):
    """Each group of channels is normalised on its own: o = (3, 4, 30, 40) in
    groups of 2 has rms 5/sqrt(2) and 50/sqrt(2), so with eps = 0 and a large
    gate (silu(40) = 40 up to 4e-16) y / 40 = sqrt(2) (0.6, 0.8, 0.6, 0.8)."""
    o = np.array([[3.0, 4.0, 30.0, 40.0]])
    z = np.full_like(o, 40.0)
    y = norm_gate(o, z, eps=0.0, group=2)
    ref = math.sqrt(2.0) * np.array([[0.6, 0.8, 0.6, 0.8]]) * 40.0
    # whole-width group: rms = sqrt((9 + 16 + 900 + 1600) / 4) = sqrt(631.25)
    yw = norm_gate(o, z, eps=0.0)
    refw = o / math.sqrt(631.25) * 40.0
    return [("groups of 2", rel(y, ref), 1e-15), ("one group", rel(yw, refw), 1e-15)]


def pin_weight_per_channel(norm_gate, silu):
    """The weight scales channel c of the whole last axis, also across groups."""
    rng = np.random.default_rng(2)
    o = rng.standard_normal((3, 2, 8))
    z = rng.standard_normal((3, 2, 8))
    w = rng.standard_normal(8) + 2.0
    y1 = norm_gate(o, z, eps=1e-3, group=4)
    yw = norm_gate(o, z, weight=w, eps=1e-3, group=4)
    return [("weight is per channel", rel(yw, y1 * w), 1e-15)]


def pin_invariants(norm_gate, silu):
    """With eps = 0: y does not change when o is scaled by a positive factor,
    flips sign with o, and y / silu(z) has mean square 1 over every group."""
    rng = np.random.default_rng(3)
    o = rng.standard_normal((4, 3, 32))
    z = rng.standard_normal((4, 3, 32))
    y = norm_gate(o, z, eps=0.0, group=16)
    out = [("scale 1e3", rel(norm_gate(o * 1e3, z, eps=0.0, group=16), y), 1e-14),
           ("scale 1e-3", rel(norm_gate(o * 1e-3, z, eps=0.0, group=16), y), 1e-14),
           ("odd in o", rel(norm_gate(-o, z, eps=0.0, group=16), -y), 1e-15)]
    u = (y / silu(z)).reshape(-1, 16)
    out.append(("unit mean square", float(np.abs(np.mean(u * u, axis=1) - 1.0).max()), 1e-13))
    return out


def pin_eps(norm_gate, silu):
    """A zero group stays zero for eps > 0; a constant group c gives
    c / sqrt(c^2 + eps) times the gate."""
    z = np.array([[1.5, -0.5, 2.0, 0.25]])
    y0 = norm_gate(np.zeros((1, 4)), z, eps=1e-6)
    c = 0.01
    yc = norm_gate(np.full((1, 4), c), z, eps=1e-4)
    ref = c / math.sqrt(c * c + 1e-4) * silu(z)
    err0 = float(np.abs(y0).max()) if np.all(np.isfinite(y0)) else math.inf
    return [("zero group", err0, 0.0), ("constant group with eps", rel(yc, ref), 1e-15)]


ALL_PINS = [pin_golden, pin_silu, pin_groups, pin_weight_per_channel, pin_invariants, pin_eps]
