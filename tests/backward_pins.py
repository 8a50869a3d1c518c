"""Pins for the fp64 backward oracle (reverse-mode differentiation of the
Gated Delta Rule-2 recurrence).

Each pin is ``pin_x(bwd) -> list[(label, err, tol)]`` with ``bwd`` following
the :func:`oracle.bwd` contract, so the same checks run against the oracle and
against deliberately broken copies of it.  The facts come from the definition
of the derivative (central finite differences of the forward oracle, which is
pinned on its own), from an independent fp64 rendering of the pages'
chunkwise backward equations, and from a closed form.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import chunk_ref
from tests.oracle_pins import rand_inputs, rel

NAMES = ("q", "k", "v", "g", "b", "w")


def _case(seed, B, T, H, dk, dv, bscale=2.0):
    q, k, v, g, b, w = rand_inputs(seed, B, T, H, dk, dv, bscale=bscale)
    rng = np.random.default_rng(seed + 100)
    N = B
    S0 = rng.standard_normal((N, H, dk, dv))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    return [q, k, v, g, b, w], S0, dO, dST


def pin_finite_differences(bwd):
    """Every gradient against central differences of L = sum(dO * o) +
    sum(dST * S_T), h = 1e-6 (truncation error ~1e-10 relative)."""
    out = []
    for seed, (B, T, H, dk, dv) in ((1, (1, 9, 1, 3, 2)), (2, (2, 5, 2, 2, 3))):
        xs, S0, dO, dST = _case(seed, B, T, H, dk, dv)
        gr = bwd(*xs, dO, S0=S0, dST=dST)

        def loss(args, s0):
            o, ST = oracle.fwd(*args, S0=s0)
            return float((o * dO).sum() + (ST * dST).sum())
        h = 1e-6
        for ai, nm in enumerate(NAMES + ("S0",)):
            base = xs[ai] if ai < 6 else S0
            fd = np.zeros_like(base)
            for idx in np.ndindex(base.shape):
                vals = []
                for sgn in (1, -1):
                    args = [x.copy() for x in xs]
                    s0 = S0.copy()
                    (args[ai] if ai < 6 else s0)[idx] += sgn * h
                    vals.append(loss(args, s0))
                fd[idx] = (vals[0] - vals[1]) / (2 * h)
            out.append((f"seed {seed} d{nm} vs finite differences", rel(gr["d" + nm], fd), 1e-7))
    return out


def pin_chunkwise(bwd):
    """The pages' chunkwise backward (fp64 numpy, chunks of 64, 17 and 1,
    including partial chunks and packed sequences) gives the same gradients."""
    out = []
    xs, S0, dO, dST = _case(3, 2, 150, 2, 8, 6)
    gr = bwd(*xs, dO, S0=S0, dST=dST)
    for C in (64, 17, 1):
        ref = chunk_ref.bwd(*xs, dO, S0=S0, dST=dST, C=C)
        out.append((f"chunk {C}", max(rel(gr[n], ref[n]) for n in ref), 1e-12))
    lens = [7, 1, 0, 70, 22]
    cu = np.concatenate([[0], np.cumsum(lens)])
    xs, _, dO, _ = _case(4, 1, int(cu[-1]), 2, 8, 6)
    S0 = np.random.default_rng(5).standard_normal((len(lens), 2, 8, 6))
    dST = np.random.default_rng(6).standard_normal((len(lens), 2, 8, 6))
    gr = bwd(*xs, dO, S0=S0, dST=dST, cu_seqlens=cu)
    ref = chunk_ref.bwd(*xs, dO, S0=S0, dST=dST, cu_seqlens=cu, C=64)
    out.append(("packed sequences", max(rel(gr[n], ref[n]) for n in ref), 1e-12))
    return out


def pin_linear_attention(bwd):
    """b = 0, g = 0, w = 1 is plain linear attention, o_t = S0^T q_t +
    sum_{s <= t} (q_t . k_s) v_s, whose gradients are written out here."""
    xs, S0, dO, dST = _case(7, 1, 12, 1, 4, 3)
    q, k, v = xs[0][0, :, 0], xs[1][0, :, 0], xs[2][0, :, 0]
    g = np.zeros((1, 12, 1, 4))
    b = np.zeros((1, 12, 1, 4))
    w = np.ones((1, 12, 1, 3))
    do, s0, dst = dO[0, :, 0], S0[0, 0], dST[0, 0]
    gr = bwd(xs[0], xs[1], xs[2], g, b, w, dO, S0=S0, dST=dST)
    T = q.shape[0]
    causal = np.tril(np.ones((T, T)))                    # [t, s] = 1 for s <= t
    P = (do @ v.T) * causal                              # [t, s] = v_s . do_t
    dq = P @ k + do @ s0.T
    dk = P.T @ q + v @ dst.T
    dv = ((q @ k.T) * causal).T @ do + k @ dst
    dS0 = q.T @ do + dst
    return [("linear attention dq", rel(gr["dq"][0, :, 0], dq), 1e-13),
            ("linear attention dk", rel(gr["dk"][0, :, 0], dk), 1e-13),
            ("linear attention dv", rel(gr["dv"][0, :, 0], dv), 1e-13),
            ("linear attention dS0", rel(gr["dS0"][0, 0], dS0), 1e-13)]


ALL_PINS = [pin_finite_differences, pin_chunkwise, pin_linear_attention]
