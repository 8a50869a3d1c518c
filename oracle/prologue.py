"""fp64 numpy oracle of the gate prologue and grouped value heads (test
infrastructure).

Gated DeltaNet-2 pages:
* "Gate Parameterization", Eq. 12: the log-decay g = -exp(a) * softplus(f + delta),
  with f = W_f x the decay branch's projection, a and delta learnable per key
  channel, alpha = exp(g), all in fp32 on the pages.
* Eq. 11: the erase gate b = sigmoid(W_b x), scaled by 2 for the
  negative-eigenvalue variant, and the write gate w = sigmoid(W_w x).
* "Big-Picture Architecture" item 1 and the token-mixer block item 2: q and k
  are L2-normalised per head.
* Grouped-value heads: with H_v = G * H value heads, the key-side tensors q,
  k, g and b are repeated across each group of value heads; v and w live on
  the value-head axis.

Readings where the pages leave a step open: a and delta are per (key head,
key channel), shape [H, dk]; the L2 norm is x / sqrt(sum(x^2) + eps) over the
dk channels of one (token, head); the value heads of one group are
consecutive, so value head h_v reads key head h_v // G.

Inputs are converted exactly to fp64; every result is fp64.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def softplus(x):
    """log(1 + e^x), evaluated without overflow."""
    return np.logaddexp(0.0, _f64(x))


def sigmoid(x):
    x = _f64(x)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def log_decay(f, a, delta):
    """Eq. 12: g = -exp(a) * softplus(f + delta); a, delta broadcast over the
    leading axes of f ([..., H, dk] against [H, dk])."""
    f, a, delta = _f64(f), _f64(a), _f64(delta)
    return -np.exp(a) * softplus(f + delta)


def l2_normalize(x, eps: float):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))


def expand_heads(x, group: int):
    """Key-side tensor [..., H, d] -> [..., H * group, d]; value head h_v gets
    key head h_v // group."""
    return np.repeat(_f64(x), int(group), axis=-2)


def block_inputs(q, k, v, f, b, w, a=None, delta=None, *, b_scale: float = 1.0,
                 qk_eps: float = 1e-6, qk_norm: bool = True, decay: bool = True,
                 gates: bool = True, value_heads: int | None = None):
    """The operator's inputs from the block's stored tensors.

    q, k, f, b: [B, T, H, dk] (f is W_f x when ``decay``, else the log-decay
    itself; b is W_b x when ``gates``, else the erase gate); v, w: [B, T, H_v,
    dv] (w is W_w x when ``gates``).  Returns (q, k, v, g, b, w) with the
    key-side tensors expanded to H_v heads, ready for :func:`oracle.fwd`."""
    q, k, v, f, b, w = (_f64(x) for x in (q, k, v, f, b, w))
    H = q.shape[-2]
    Hv = v.shape[-2] if value_heads is None else int(value_heads)
    assert Hv % H == 0, "value heads must be a multiple of key heads"
    if qk_norm:
        q, k = l2_normalize(q, qk_eps), l2_normalize(k, qk_eps)
    g = log_decay(f, a, delta) if decay else f
    if gates:
        b = b_scale * sigmoid(b)
        w = sigmoid(w)
    grp = Hv // H
    q, k, g, b = (expand_heads(x, grp) for x in (q, k, g, b))
    return q, k, v, g, b, w
