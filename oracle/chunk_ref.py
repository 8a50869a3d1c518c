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
