"""fp64 numpy oracle of the output epilogue (test infrastructure).

Gated DeltaNet-2 pages, "Big-Picture Architecture" item 6 and "Gated
DeltaNet-2 token mixer block" item 5: the recurrent output o is RMS-normalised
and then multiplied channel by channel by a SiLU-activated output gate.

The pages name the two operations and their order but not the normalisation
width, the epsilon or the weight.  The reading taken here: the usual RMSNorm
of the Gated DeltaNet family,

    y = o / sqrt(mean(o^2) + eps) * weight * silu(z),    silu(z) = z * sigmoid(z),

with the mean taken over consecutive groups of ``group`` channels of the last
axis (``group = dv`` normalises each head on its own, ``group = H*dv`` the
whole token), eps >= 0 inside the square root, and an optional per-channel
weight along the whole last axis.  z, the gate's pre-activation, has the shape
of o.

Inputs are converted exactly to fp64; the result is fp64.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def norm_gate(o, z, weight=None, eps: float = 1e-6, group: int | None = None):
    """RMSNorm of each ``group``-channel group of o's last axis, times the
    per-channel ``weight`` (None: ones) and silu(z)."""
    o, z = _f64(o), _f64(z)
    assert o.shape == z.shape, "o and z must have one shape"
    d = o.shape[-1]
    group = d if group is None else int(group)
    assert group > 0 and d % group == 0, "group must divide the last axis"
    g = o.reshape(-1, d // group, group)
    mean_sq = np.mean(g * g, axis=-1, keepdims=True)
    y = (g / np.sqrt(mean_sq + float(eps))).reshape(o.shape)
    if weight is not None:
        w = _f64(weight)
        assert w.shape == (d,), "weight has one entry per channel of the last axis"
        y = y * w
    return y * silu(z)
