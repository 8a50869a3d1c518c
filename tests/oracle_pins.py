"""Pins for the fp64 oracle: facts the Gated DeltaNet-2 pages and plain
mathematics fix, independent of the oracle's own code.

Every pin is a function ``pin_x(fwd, decode) -> list[(label, err, tol)]`` so the
same checks run against the real oracle (tests/test_oracle_pins.py) and against
deliberately broken copies of it (the mutation test), which must each fail at
least one pin.  ``fwd``/``decode`` follow the :mod:`oracle` calling contract.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from oracle import chunk_ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rel(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


def rand_inputs(seed, B, T, H, dk, dv, shift=0.0, bscale=1.0, unit=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H, dk)) + shift))
    b = bscale / (1 + np.exp(-rng.standard_normal((B, T, H, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, dv))))
    return q, k, v, g, b, w


# -- golden: a hand-worked two-token example (tests/golden) ----------------------

def pin_golden(fwd, decode):
    with open(os.path.join(GOLDEN, "hand_worked_dk2_dv2.json")) as f:
        gd = json.load(f)
    toks = gd["tokens"]
    arr = lambda key: np.array([t[key] for t in toks], np.float64)[None, :, None, :]
    q, k, v, b, w = arr("q"), arr("k"), arr("v"), arr("b"), arr("w")
    g = np.log(arr("alpha"))
    S0 = np.array(gd["S0"], np.float64)[None, None]
    o, ST = fwd(q, k, v, g, b, w, S0=S0)
    return [("golden o", rel(o[0, :, 0], gd["expected_o"]), 1e-14),
            ("golden S_T", rel(ST[0, 0], gd["expected_S_T"]), 1e-14)]


# -- P1: the pages' chunkwise WY algorithm equals the recurrence -----------------

def pin_chunkwise(fwd, decode):
    out = []
    for seed, shift, bscale in ((1, 0.0, 1.0), (2, -2.0, 2.0)):
        q, k, v, g, b, w = rand_inputs(seed, 2, 150, 2, 16, 8, shift, bscale)
        S0 = 0.1 * np.random.default_rng(seed + 10).standard_normal((2, 2, 16, 8))
        o, ST = fwd(q, k, v, g, b, w, S0=S0)
        for C in (64, 17, 1):
            oc, STc = chunk_ref.fwd(q, k, v, g, b, w, S0=S0, C=C)
            out.append((f"chunkwise C={C} o (seed {seed})", rel(o, oc), 1e-12))
            out.append((f"chunkwise C={C} S_T (seed {seed})", rel(ST, STc), 1e-12))
    return out


# -- P2/P3: collapse to KDA and Gated DeltaNet -----------------------------------

def _kda(q, k, v, alpha, beta, S0):
    """Kimi Delta Attention written from its own form (pages, related work:
    S_t = (I - beta k k^T) Diag(alpha) S + beta k v^T)."""
    S = S0.copy()
    o = np.zeros((q.shape[0], v.shape[1]))
    I = np.eye(q.shape[1])
    for t in range(q.shape[0]):
        S = (I - beta[t] * np.outer(k[t], k[t])) @ (alpha[t][:, None] * S) \
            + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def _gdn(q, k, v, alpha, beta, S0):
    """Gated DeltaNet (scalar decay): S_t = alpha (I - beta k k^T) S + beta k v^T."""
    S = S0.copy()
    o = np.zeros((q.shape[0], v.shape[1]))
    I = np.eye(q.shape[1])
    for t in range(q.shape[0]):
        S = alpha[t] * ((I - beta[t] * np.outer(k[t], k[t])) @ S) + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def pin_collapses(fwd, decode):
    out = []
    T, dk, dv = 40, 6, 5
    q, k, v, g, _, _ = rand_inputs(3, 1, T, 1, dk, dv)
    rng = np.random.default_rng(4)
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((dk, dv))
    b = np.broadcast_to(beta[None, :, None, None], (1, T, 1, dk)).copy()
    w = np.broadcast_to(beta[None, :, None, None], (1, T, 1, dv)).copy()
    o, ST = fwd(q, k, v, g, b, w, S0=S0[None, None])
    ok, Sk = _kda(q[0, :, 0], k[0, :, 0], v[0, :, 0], np.exp(g[0, :, 0]), beta, S0)
    out += [("KDA collapse o", rel(o[0, :, 0], ok), 1e-12), ("KDA collapse S_T", rel(ST[0, 0], Sk), 1e-12)]
    gs = -np.log1p(np.exp(rng.standard_normal(T)))
    g2 = np.broadcast_to(gs[None, :, None, None], (1, T, 1, dk)).copy()
    o, ST = fwd(q, k, v, g2, b, w, S0=S0[None, None])
    og, Sg = _gdn(q[0, :, 0], k[0, :, 0], v[0, :, 0], np.exp(gs), beta, S0)
    out += [("GDN collapse o", rel(o[0, :, 0], og), 1e-12), ("GDN collapse S_T", rel(ST[0, 0], Sg), 1e-12)]
    return out


# -- P4: read-after-write; P5: pure decay -----------------------------------------

def pin_read_after_write(fwd, decode):
    q, k, v, g, b, w = rand_inputs(5, 1, 30, 2, 8, 6)
    S0 = np.random.default_rng(6).standard_normal((1, 2, 8, 6))
    o, _ = fwd(k, k, v, np.zeros_like(g), np.ones_like(b), w, S0=S0)   # q_t = k_t
    return [("read after write S_t^T k_t = w*v", rel(o, w * v), 1e-13)]


def pin_pure_decay(fwd, decode):
    q, k, v, g, b, w = rand_inputs(7, 1, 25, 2, 8, 6, shift=-1.0)
    S0 = np.random.default_rng(8).standard_normal((1, 2, 8, 6))
    o, ST = fwd(q, k, v, g, np.zeros_like(b), np.zeros_like(w), S0=S0)
    G = np.cumsum(g[0], axis=0)                                  # [T, H, dk]
    St = np.exp(G)[..., None] * S0[0][None]                      # [T, H, dk, dv]
    o_ref = np.einsum("thij,thi->thj", St, q[0])
    return [("pure decay S_T", rel(ST[0], St[-1]), 1e-13), ("pure decay o", rel(o[0], o_ref), 1e-13)]


# -- P6: brute-force transition products on tiny inputs ---------------------------

def pin_bruteforce(fwd, decode):
    out = []
    T, dk, dv = 9, 3, 5
    q, k, v, g, b, w = rand_inputs(9, 1, T, 1, dk, dv, bscale=2.0, unit=False)
    S0 = np.random.default_rng(10).standard_normal((dk, dv))
    o, ST = fwd(q, k, v, g, b, w, S0=S0[None, None])
    q, k, v, g, b, w = (x[0, :, 0] for x in (q, k, v, g, b, w))
    M = [(np.eye(dk) - np.outer(k[t], b[t] * k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    def prod(lo, hi):  # M_{hi-1} ... M_lo
        P = np.eye(dk)
        for t in range(lo, hi):
            P = M[t] @ P
        return P
    o_ref = np.zeros((T, dv))
    for t in range(T):
        St = prod(0, t + 1) @ S0 + sum(prod(s + 1, t + 1) @ np.outer(k[s], w[s] * v[s])
                                       for s in range(t + 1))
        o_ref[t] = St.T @ q[t]
    out += [("brute-force product S_T", rel(ST[0, 0], St), 1e-13),
            ("brute-force product o", rel(o[0, :, 0], o_ref), 1e-13)]
    # exact rational arithmetic on a 3-token dk=2, dv=3 case (alpha = 1/2, 3/4)
    al = [[Fraction(1, 2), Fraction(3, 4)], [Fraction(3, 4), Fraction(1)], [Fraction(1), Fraction(1, 2)]]
    kk = [[Fraction(1), Fraction(2)], [Fraction(-1), Fraction(1, 3)], [Fraction(2, 5), Fraction(1)]]
    bb = [[Fraction(1, 2), Fraction(3, 2)], [Fraction(1), Fraction(1, 4)], [Fraction(2), Fraction(0)]]
    ww = [[Fraction(1), Fraction(1, 2), Fraction(0)], [Fraction(1, 4), Fraction(1), Fraction(1)],
          [Fraction(1, 2), Fraction(1, 2), Fraction(1, 2)]]
    vv = [[Fraction(1), Fraction(-2), Fraction(3)], [Fraction(0), Fraction(1), Fraction(-1)],
          [Fraction(2), Fraction(2), Fraction(-3)]]
    qq = [[Fraction(1), Fraction(0)], [Fraction(1, 2), Fraction(1, 2)], [Fraction(-1), Fraction(3)]]
    S = [[Fraction(1), Fraction(0), Fraction(-1)], [Fraction(2), Fraction(1, 2), Fraction(0)]]
    S0f = [row[:] for row in S]
    o_ex = []
    for t in range(3):
        # S_t = (I - k e^T) D S + k z^T written as explicit 2x2 transition matrix times S
        Mt = [[(1 if i == r else 0) - kk[t][i] * bb[t][r] * kk[t][r] for r in range(2)] for i in range(2)]
        Mt = [[Mt[i][r] * al[t][r] for r in range(2)] for i in range(2)]
        S = [[sum(Mt[i][r] * S[r][j] for r in range(2)) + kk[t][i] * ww[t][j] * vv[t][j]
              for j in range(3)] for i in range(2)]
        o_ex.append([sum(S[i][j] * qq[t][i] for i in range(2)) for j in range(3)])
    f = lambda a: np.array([[float(x) for x in row] for row in a])[None, :, None, :]
    o2, ST2 = fwd(f(qq), f(kk), f(vv), np.log(f(al)), f(bb), f(ww),
                  S0=np.array([[float(x) for x in row] for row in S0f])[None, None])
    out += [("exact rational o", rel(o2[0, :, 0], [[float(x) for x in r] for r in o_ex]), 1e-14),
            ("exact rational S_T", rel(ST2[0, 0], [[float(x) for x in r] for r in S]), 1e-14)]
    return out


# -- P7: Householder endpoint of the negative-eigenvalue range ---------------------

def pin_householder(fwd, decode):
    T, dk, dv = 12, 6, 4
    q, k, v, g, b, w = rand_inputs(11, 1, T, 1, dk, dv)
    S0 = np.random.default_rng(12).standard_normal((1, 1, dk, dv))
    zeros_g, twos, zeros_w = np.zeros_like(g), 2 * np.ones_like(b), np.zeros_like(w)
    _, ST = fwd(q, k, v, zeros_g, twos, zeros_w, S0=S0)
    norm_err = abs(np.linalg.norm(ST) - np.linalg.norm(S0)) / np.linalg.norm(S0)
    kk = np.repeat(k[:, :1], 2, axis=1)                          # the same key twice
    _, ST2 = fwd(q[:, :2], kk, v[:, :2], zeros_g[:, :2], twos[:, :2], zeros_w[:, :2], S0=S0)
    return [("reflector keeps ||S||_F", norm_err, 1e-13), ("reflector twice restores S", rel(ST2, S0), 1e-13)]


# -- P8: linearity in (S0, v) and channel equivariance -------------------------------

def pin_linearity(fwd, decode):
    q, k, v1, g, b, w = rand_inputs(13, 1, 35, 2, 8, 6, bscale=2.0)
    rng = np.random.default_rng(14)
    v2 = rng.standard_normal(v1.shape)
    S1, S2 = rng.standard_normal((2, 1, 2, 8, 6))
    a1, a2 = 0.7, -1.3
    o1, T1 = fwd(q, k, v1, g, b, w, S0=S1)
    o2, T2 = fwd(q, k, v2, g, b, w, S0=S2)
    o3, T3 = fwd(q, k, a1 * v1 + a2 * v2, g, b, w, S0=a1 * S1 + a2 * S2)
    out = [("superposition o", rel(o3, a1 * o1 + a2 * o2), 1e-12),
           ("superposition S_T", rel(T3, a1 * T1 + a2 * T2), 1e-12)]
    pv = rng.permutation(6)
    o4, T4 = fwd(q, k, v1[..., pv], g, b, w[..., pv], S0=S1[..., pv])
    out += [("dv permutation o", rel(o4, o1[..., pv]), 1e-13), ("dv permutation S_T", rel(T4, T1[..., pv]), 1e-13)]
    pk = rng.permutation(8)
    o5, T5 = fwd(q[..., pk], k[..., pk], v1, g[..., pk], b[..., pk], w, S0=S1[:, :, pk])
    out += [("dk permutation o", rel(o5, o1), 1e-12), ("dk permutation S_T", rel(T5, T1[:, :, pk]), 1e-12)]
    return out


# -- P9: fast-weight stationarity (pages, Eq. 13 and its gradient) -----------------

def pin_fast_weight(fwd, decode):
    q, k, v, g, b, w = rand_inputs(15, 1, 1, 1, 7, 5, bscale=2.0)
    S0 = np.random.default_rng(16).standard_normal((7, 5))
    _, ST = fwd(q, k, v, g, b, w, S0=S0[None, None])
    St = ST[0, 0]
    kt, et, zt = k[0, 0, 0], (b * k)[0, 0, 0], (w * v)[0, 0, 0]
    Sbar = np.exp(g[0, 0, 0])[:, None] * S0
    L = lambda S: np.sum((S - Sbar) ** 2) - 2 * np.dot(S.T @ kt, zt - Sbar.T @ et)
    # L is quadratic with Hessian 2I: L(S* + D) - L(S*) = ||D||^2 iff S* is its minimiser
    rng = np.random.default_rng(17)
    errs = []
    for _ in range(5):
        D = rng.standard_normal(St.shape)
        errs.append(abs(L(St + D) - L(St) - np.sum(D ** 2)) / np.sum(D ** 2))
    rank = np.linalg.matrix_rank(St - Sbar, tol=1e-10)
    return [("fast-weight minimiser", max(errs), 1e-12), ("rank-1 edit", float(rank != 1), 0.0)]


# -- P10: the scalar case dk = 1 ---------------------------------------------------

def pin_scalar(fwd, decode):
    T, dv = 20, 4
    q, k, v, g, b, w = rand_inputs(18, 1, T, 1, 1, dv, unit=False, bscale=2.0)
    S0 = np.random.default_rng(19).standard_normal((1, 1, 1, dv))
    o, ST = fwd(q, k, v, g, b, w, S0=S0)
    s = S0[0, 0, 0].copy()
    o_ref = np.zeros((T, dv))
    for t in range(T):
        kt, bt, at = k[0, t, 0, 0], b[0, t, 0, 0], np.exp(g[0, t, 0, 0])
        s = (1 - bt * kt * kt) * at * s + kt * w[0, t, 0] * v[0, t, 0]
        o_ref[t] = s * q[0, t, 0, 0]
    return [("dk=1 closed form o", rel(o[0, :, 0], o_ref), 1e-14), ("dk=1 closed form S_T", rel(ST[0, 0, 0], s), 1e-14)]


# -- P11: composition (state passing, varlen reset, decode = forward) -------------

def pin_composition(fwd, decode):
    out = []
    q, k, v, g, b, w = rand_inputs(20, 1, 60, 2, 8, 6, bscale=2.0)
    S0 = np.random.default_rng(21).standard_normal((1, 2, 8, 6))
    o, ST = fwd(q, k, v, g, b, w, S0=S0)
    t1 = 23
    oa, Sa = fwd(*(x[:, :t1] for x in (q, k, v, g, b, w)), S0=S0)
    ob, Sb = fwd(*(x[:, t1:] for x in (q, k, v, g, b, w)), S0=Sa)
    out += [("split/resume o", rel(np.concatenate([oa, ob], 1), o), 1e-13), ("split/resume S_T", rel(Sb, ST), 1e-13)]
    lens = [7, 1, 30, 22]
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0v = np.random.default_rng(22).standard_normal((4, 2, 8, 6))
    ov, Sv = fwd(q, k, v, g, b, w, S0=S0v, cu_seqlens=cu)
    err_o = err_s = 0.0
    for n in range(4):
        sl = slice(int(cu[n]), int(cu[n + 1]))
        on, Sn = fwd(*(x[:, sl] for x in (q, k, v, g, b, w)), S0=S0v[n:n + 1])
        err_o = max(err_o, rel(ov[:, sl], on))
        err_s = max(err_s, rel(Sv[n], Sn[0]))
    out += [("varlen = separate o", err_o, 1e-13), ("varlen = separate S_T", err_s, 1e-13)]
    S = S0[0][None].copy()   # decode batch of one sequence
    od = np.zeros_like(o)
    for t in range(60):
        step = [x[:, t] for x in (q, k, v, g, b, w)]
        od[:, t], S = decode(*step, S)
    out += [("decode x T = forward o", rel(od, o), 1e-13), ("decode x T = forward S", rel(S, ST), 1e-13)]
    return out


ALL_PINS = [pin_golden, pin_chunkwise, pin_collapses, pin_read_after_write, pin_pure_decay,
            pin_bruteforce, pin_householder, pin_linearity, pin_fast_weight, pin_scalar,
            pin_composition]
