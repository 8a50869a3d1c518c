"""Error metrics for comparing the GPU path with the fp64 oracle.

Tolerances (written in the tests that use them):
* fp32 path: max relative error per tensor, ``max|x - ref| / max|ref| <= 1e-4``.
* bf16 path: max-abs error normalised by the reference RMS, ``<= 2e-2`` on o and
  S_T.  o is stored in bf16, whose own rounding of an exact value already costs
  up to half a bf16 ulp; that storage rounding is granted element by element
  and the 2e-2 bound applies to the error the arithmetic adds on top of it
  (:func:`bf16_excess`).  S_T is fp32 and gets no allowance.
"""
from __future__ import annotations

import numpy as np


def as64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def max_rel(x, ref) -> float:
    x, ref = as64(x), as64(ref)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-300))


def rms(ref) -> float:
    ref = as64(ref)
    return float(np.sqrt(np.mean(ref * ref)))


def rms_err(x, ref) -> float:
    x, ref = as64(x), as64(ref)
    return float(np.abs(x - ref).max() / max(rms(ref), 1e-300))


def bf16_half_ulp(ref) -> np.ndarray:
    """Half the bf16 spacing at each |ref| (0 for ref == 0)."""
    ref = as64(ref)
    _, e = np.frexp(ref)               # |ref| = m * 2**e, m in [0.5, 1)
    h = np.ldexp(1.0, e - 9)           # bf16 keeps 8 significant bits
    return np.where(ref == 0, 0.0, h)


def bf16_excess(x, ref) -> float:
    x, ref = as64(x), as64(ref)
    ex = np.maximum(np.abs(x - ref) - bf16_half_ulp(ref), 0.0)
    return float(ex.max() / max(rms(ref), 1e-300))
