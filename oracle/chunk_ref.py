"""fp64 numpy rendering of the pages' chunkwise WY algorithm (test infrastructure).

Gated DeltaNet-2 pages, "Chunkwise Parallel Training via WY Representation":
Step 1 (decay-normalised state, cumulative log-decay G and gamma = exp(G)),
Step 2 (chunk matrices of Eq. 20, the strictly lower triangular T, the WY
inverse A = (I + T)^-1 and the auxiliaries Y = A E_bar, U = A Z), Step 3
(state and output equations, Eqs. 23-24).

It exists to pin the token-by-token oracle: the chunkwise form is an exact
reformulation of Eq. 10, so both must agree to fp64 rounding for every chunk
size, including chunks that end part-way and C = 1.  It also exposes the
per-chunk intermediates (T, A, Y, U, A_qk) for inspecting GPU tiles.  Library
primitives used: cumulative sum, exp, matrix product and a unit lower
triangular solve (the pages' forward substitution).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_step(S0, q, k, v, g, b, w, keep: bool = False):
    """Advance one chunk.  q, k, g, b: [C, dk]; v, w: [C, dv]; S0: [dk, dv].
    Returns (O [C, dv], S_C [dk, dv], intermediates or None)."""
    C = q.shape[0]
    G = np.cumsum(g, axis=0)                      # G_r = sum_{i<=r} g_i  (Step 1)
    gam = np.exp(G)                               # gamma_r, gamma_0 = 1 implicit
    Kbar = k / gam                                # k_bar_r = gamma_r^-1 * k_r
    Ebar = gam * (b * k)                          # e_bar_r = gamma_r * (b_r * k_r)   (Eq. 20)
    Z = w * v                                     # z_r = w_r * v_r                   (Eq. 20)
    T = np.tril(Ebar @ Kbar.T, -1)                # T_rs = e_bar_r . k_bar_s, s < r
    A = solve_triangular(np.eye(C) + T, np.eye(C), lower=True, unit_diagonal=True)
    Y = A @ Ebar                                  # WY auxiliaries
    U = A @ Z
    gC = gam[-1]
    Ktail = (gC / gam) * k                        # row r: (gamma_C / gamma_r) * k_r
    Qg = gam * q                                  # row r: gamma_r * q_r
    # (A_qk)_rs = 1[r >= s] q_r^T Diag(gamma_r / gamma_s) k_s
    ratio = np.exp(G[:, None, :] - G[None, :, :])            # [r, s, i]
    Aqk = np.einsum("ri,rsi,si->rs", q, ratio, k)
    Aqk = np.tril(Aqk, 0)
    R = U - Y @ S0                                # chunk-local residual
    O = Qg @ S0 + Aqk @ R                         # Eq. 24
    SC = gC[:, None] * S0 + Ktail.T @ R           # Eq. 23
    inter = dict(G=G, T=T, A=A, Y=Y, U=U, Aqk=Aqk, Qg=Qg, Ktail=Ktail) if keep else None
    return O, SC, inter


def fwd_head(q, k, v, g, b, w, S0, C: int = 64):
    """One (sequence, head): q, k, g, b [L, dk]; v, w [L, dv]; S0 [dk, dv].
    Chunks of C tokens from the sequence start; the last one may be short."""
    L = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((L, v.shape[1]), dtype=np.float64)
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        O, S, _ = chunk_step(S, q[sl], k[sl], v[sl], g[sl], b[sl], w[sl])
        o[sl] = O
    return o, S


def fwd(q, k, v, g, b, w, S0=None, cu_seqlens=None, C: int = 64):
    """Same contract as :func:`oracle.fwd` (fp64 arrays [B, T, H, d])."""
    q, k, v, g, b, w = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b, w))
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    flat = [x.reshape(Bsz * T, H, -1) for x in (q, k, v, g, b, w)]
    cu = (np.arange(Bsz + 1) * T if cu_seqlens is None
          else np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.size - 1
    o = np.zeros((Bsz * T, H, dv))
    ST = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)[n, h]
            sl = slice(int(cu[n]), int(cu[n + 1]))
            args = [x[sl, h] for x in flat]
            o[sl, h], ST[n, h] = fwd_head(*args, s0, C=C)
    return o.reshape(Bsz, T, H, dv), ST


# -- backward -------------------------------------------------------------------------
#
# Gated DeltaNet-2 pages, "Gate-Aware Backward Pass" (Appendix B): the output and
# state paths first (the state and output equations differentiated, chunks in
# reverse), then the gate-aware WY inverse path (Eqs. 64-65: dA gets dU Z^T and
# dY E_bar^T with the gates inside the products), the triangular inverse VJP
# dT = -tril(A^T dA A^T, -1), dE_bar and dK_bar from T = E_bar K_bar^T, and the
# elementwise gate products, ending with the reverse cumulative sum that turns
# dgamma into dg (Step 4 of the backward flow).

def chunk_backward(S0, q, k, v, g, b, w, dO, dSC):
    """One chunk: entry state S0 [dk, dv], inputs as chunk_step, dO [C, dv],
    dSC = dL/d(exit state).  Returns (grads dict over q, k, v, g, b, w with
    chunk rows, dL/dS0, intermediates dict)."""
    C = q.shape[0]
    _, _, it = chunk_step(S0, q, k, v, g, b, w, keep=True)
    G, A, Y, U, Aqk, Qg, Ktail = (it[x] for x in ("G", "A", "Y", "U", "Aqk", "Qg", "Ktail"))
    gam = np.exp(G)
    gC = gam[-1]
    Kbar = k / gam
    Ebar = gam * (b * k)
    Z = w * v
    # output and state paths: O = Qg S + Aqk R, S' = Diag(gC) S + Ktail^T R, R = U - Y S
    R = U - Y @ S0
    dR = Aqk.T @ dO + Ktail @ dSC
    dQg = dO @ S0.T
    dAqk = np.tril(dO @ R.T, 0)
    dKtail = R @ dSC.T
    dgC = np.sum(dSC * S0, axis=1)
    dS0 = Qg.T @ dO + gC[:, None] * dSC - Y.T @ dR
    dU, dY = dR, -dR @ S0.T
    # gate-aware WY inverse path (Eqs. 64-65)
    dA = dU @ Z.T + dY @ Ebar.T
    dZ = A.T @ dU
    dEbar = A.T @ dY
    dT = -np.tril(A.T @ dA @ A.T, -1)
    dEbar += dT @ Kbar
    dKbar = dT.T @ Ebar
    # A_qk = tril(Qg Kbar^T, 0)
    dQg += dAqk @ Kbar
    dKbar += dAqk.T @ Qg
    # elementwise products and the decay
    dw, dv = dZ * v, dZ * w
    dq = dQg * gam
    dgam = dQg * q
    dk = dKbar / gam
    dgam -= dKbar * Kbar / gam
    db = dEbar * gam * k
    dk += dEbar * gam * b
    dgam += dEbar * b * k
    dk += dKtail * (gC / gam)
    dgam -= dKtail * Ktail / gam
    dgC += np.sum(dKtail * k / gam, axis=0)
    dG = dgam * gam
    dG[-1] += dgC * gC
    dg = np.cumsum(dG[::-1], axis=0)[::-1]        # dg_i = sum_{r >= i} dG_r
    grads = dict(q=dq, k=dk, v=dv, g=dg, b=db, w=dw)
    inter = dict(dR=dR, dA=dA, dT=dT, dEbar=dEbar, dKbar=dKbar, dQg=dQg, dAqk=dAqk,
                 dKtail=dKtail, dgC=dgC, dZ=dZ)
    return grads, dS0, inter


def bwd_head(q, k, v, g, b, w, S0, dO, dST, C: int = 64):
    """One (sequence, head): chunk-entry states from a forward sweep, then the
    chunks in reverse."""
    L = q.shape[0]
    starts = list(range(0, L, C))
    S = np.array(S0, dtype=np.float64, copy=True)
    entry = []
    for c0 in starts:
        entry.append(S)
        sl = slice(c0, min(L, c0 + C))
        _, S, _ = chunk_step(S, q[sl], k[sl], v[sl], g[sl], b[sl], w[sl])
    grads = {n: np.zeros_like(x) for n, x in (("q", q), ("k", k), ("v", v), ("g", g), ("b", b),
                                              ("w", w))}
    dS = np.array(dST, dtype=np.float64, copy=True)
    for c0, Sc in zip(reversed(starts), reversed(entry)):
        sl = slice(c0, min(L, c0 + C))
        gr, dS, _ = chunk_backward(Sc, q[sl], k[sl], v[sl], g[sl], b[sl], w[sl], dO[sl], dS)
        for n in grads:
            grads[n][sl] = gr[n]
    return grads, dS


def bwd(q, k, v, g, b, w, dO, S0=None, dST=None, cu_seqlens=None, C: int = 64):
    """Same contract as :func:`oracle.bwd`."""
    q, k, v, g, b, w, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, b, w, dO))
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    flat = [x.reshape(Bsz * T, H, -1) for x in (q, k, v, g, b, w, dO)]
    cu = (np.arange(Bsz + 1) * T if cu_seqlens is None
          else np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.size - 1
    out = {n: np.zeros((Bsz * T, H, dk)) for n in ("dq", "dk", "dg", "db")}
    out.update({n: np.zeros((Bsz * T, H, dv)) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)[n, h]
            dst = np.zeros((dk, dv)) if dST is None else np.asarray(dST, np.float64)[n, h]
            sl = slice(int(cu[n]), int(cu[n + 1]))
            args = [x[sl, h] for x in flat]
            gr, out["dS0"][n, h] = bwd_head(*args[:6], s0, args[6], dst, C=C)
            for nm in ("q", "k", "v", "g", "b", "w"):
                out["d" + nm][sl, h] = gr[nm]
    for nm in ("dq", "dk", "dg", "db"):
        out[nm] = out[nm].reshape(Bsz, T, H, dk)
    for nm in ("dv", "dw"):
        out[nm] = out[nm].reshape(Bsz, T, H, dv)
    return out
