"""Pins for the gate-prologue oracle (Eq. 12 log-decay, Eq. 11 gates, q/k L2
norm, grouped value heads).

Each pin is ``pin_x(P) -> list[(label, err, tol)]`` where ``P`` is the oracle
module (or a deliberately broken copy of it, each of which must fail at least
one pin).  The facts come from the pages' gate parameterisation and block
description and from plain mathematics, not from the oracle's code.
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def rel(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


def pin_softplus(P):
    """softplus(0) = ln 2, softplus(x) - softplus(-x) = x, softplus(40) = 40 and
    softplus(-40) = e^-40 to fp64 rounding (no overflow or cancellation)."""
    x = np.random.default_rng(1).standard_normal(64) * 5
    return [("softplus(0)", rel(P.softplus(np.array([0.0])), [math.log(2.0)]), 1e-16),
            ("softplus odd part", rel(P.softplus(x) - P.softplus(-x), x), 1e-14),
            ("softplus(40)", rel(P.softplus(np.array([40.0])), [40.0]), 1e-16),
            ("softplus(-40)", rel(P.softplus(np.array([-40.0])), [math.exp(-40.0)]), 1e-14)]


def pin_log_decay(P):
    """Eq. 12 closed forms: f + delta = 0 gives g = -exp(a) ln 2, so a = 0 gives
    alpha = 1/2 and a = ln 3 gives alpha = 1/8; delta shifts f; g <= 0."""
    f = np.zeros((1, 1, 2, 2))
    a = np.array([[0.0, math.log(3.0)], [0.0, 0.0]])
    d = np.array([[0.0, 0.0], [1.5, -1.5]])
    alpha = np.exp(P.log_decay(f + np.array([[0.0, 0.0], [-1.5, 1.5]]), a, d))
    rng = np.random.default_rng(2)
    fr = rng.standard_normal((3, 5, 2, 4)) * 4
    ar, dr = rng.standard_normal((2, 4)), rng.standard_normal((2, 4))
    g = P.log_decay(fr, ar, dr)
    return [("alpha closed forms", rel(alpha[0, 0], [[0.5, 0.125], [0.5, 0.5]]), 1e-15),
            ("g <= 0", float(max(g.max(), 0.0)), 0.0),
            ("a scales, delta shifts", rel(g, -np.exp(ar) * np.log1p(np.exp(fr + dr))), 1e-13)]


def pin_sigmoid(P):
    x = np.random.default_rng(3).standard_normal(64) * 5
    return [("sigmoid(0)", abs(float(P.sigmoid(np.array([0.0]))[0]) - 0.5), 0.0),
            ("sigmoid(x) + sigmoid(-x)", rel(P.sigmoid(x) + P.sigmoid(-x), np.ones_like(x)), 1e-15),
            ("sigmoid(ln 3)", rel(P.sigmoid(np.array([math.log(3.0)])), [0.75]), 1e-15)]


def pin_l2(P):
    """(3, 4) -> (0.6, 0.8); with eps = 11 the root is 6; zero stays zero; random
    rows get unit norm."""
    x = np.array([[3.0, 4.0]])
    r = np.random.default_rng(4).standard_normal((7, 3, 16))
    n = np.linalg.norm(P.l2_normalize(r, 0.0), axis=-1)
    z = P.l2_normalize(np.zeros((1, 8)), 1e-6)
    return [("(3,4)", rel(P.l2_normalize(x, 0.0), [[0.6, 0.8]]), 1e-16),
            ("eps inside the root", rel(P.l2_normalize(x, 11.0), [[0.5, 4.0 / 6.0]]), 1e-16),
            ("zero row", float(np.abs(z).max()) if np.all(np.isfinite(z)) else math.inf, 0.0),
            ("unit norm", float(np.abs(n - 1).max()), 1e-15)]


def _block_case(seed, H, group, dk=8, dv=6, T=20):
    rng = np.random.default_rng(seed)
    Hv = H * group
    q = rng.standard_normal((1, T, H, dk))
    k = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, Hv, dv))
    f = rng.standard_normal((1, T, H, dk))
    b = rng.standard_normal((1, T, H, dk))
    w = rng.standard_normal((1, T, Hv, dv))
    a = rng.standard_normal((H, dk)) * 0.5
    d = rng.standard_normal((H, dk))
    return q, k, v, f, b, w, a, d


def pin_gates(P):
    """With the activations done by hand from the pages' formulas, the block
    inputs equal the operator's inputs: b in [0, 2] with the scale 2, w in
    [0, 1], q and k of unit norm."""
    q, k, v, f, b, w, a, d = _block_case(5, 2, 1)
    qq, kk, vv, gg, bb, ww = P.block_inputs(q, k, v, f, b, w, a, d, b_scale=2.0, qk_eps=0.0)
    return [("erase gate 2 sigmoid", rel(bb, 2.0 / (1.0 + np.exp(-b))), 1e-15),
            ("write gate sigmoid", rel(ww, 1.0 / (1.0 + np.exp(-w))), 1e-15),
            ("log-decay", rel(gg, -np.exp(a) * np.log1p(np.exp(f + d))), 1e-13),
            ("|q| = 1", float(np.abs(np.linalg.norm(qq, axis=-1) - 1).max()), 1e-15),
            ("|k| = 1", float(np.abs(np.linalg.norm(kk, axis=-1) - 1).max()), 1e-15),
            ("v untouched", rel(vv, v), 0.0)]


def pin_grouped_heads(P):
    """Value heads 2h and 2h+1 read key head h (groups of consecutive value
    heads): with q zero on key head 1, value heads 2 and 3 output exactly zero
    and heads 0 and 1 do not; two value heads of one group with the same v and
    w give the same output; one value head per key head is the plain operator."""
    out = []
    q, k, v, f, b, w, a, d = _block_case(6, 2, 2)
    q[:, :, 1] = 0.0
    o, _ = oracle.fwd(*P.block_inputs(q, k, v, f, b, w, a, d, qk_eps=1e-6))
    nz = [float(np.abs(o[0, :, h]).max()) for h in range(4)]
    out.append(("heads 2, 3 read key head 1", max(nz[2], nz[3]), 0.0))
    out.append(("heads 0, 1 read key head 0", 1.0 if min(nz[0], nz[1]) > 1e-3 else math.inf, 1.0))
    q, k, v, f, b, w, a, d = _block_case(7, 2, 2)
    v[:, :, 1], w[:, :, 1] = v[:, :, 0], w[:, :, 0]
    o, ST = oracle.fwd(*P.block_inputs(q, k, v, f, b, w, a, d))
    out.append(("same v, w in a group", rel(o[0, :, 1], o[0, :, 0]) + rel(ST[0, 1], ST[0, 0]), 0.0))
    q, k, v, f, b, w, a, d = _block_case(8, 3, 1)
    o1, S1 = oracle.fwd(*P.block_inputs(q, k, v, f, b, w, a, d))
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    kn = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6)
    o2, S2 = oracle.fwd(qn, kn, v, -np.exp(a) * np.logaddexp(0, f + d), 1 / (1 + np.exp(-b)),
                        1 / (1 + np.exp(-w)))
    out.append(("one value head per key head", rel(o1, o2) + rel(S1, S2), 1e-13))
    return out


ALL_PINS = [pin_softplus, pin_log_decay, pin_sigmoid, pin_l2, pin_gates, pin_grouped_heads]
