"""Error metrics for comparing the GPU path with the fp64 oracle.

Tolerances (written in the tests that use them):
* fp32 path: max relative error per tensor, ``max|x - ref| / max|ref| <= 1e-4``.
* bf16 path: max-abs error normalised by the reference RMS, ``<= 2e-2`` on o and
  S_T (:func:`rms_err`, the plain metric).  It is applied as written to S_T
  and to o stored in fp32 (gdr2_chunk_fwd_f32_out).  When o is stored in
  bf16, its own rounding of an exact value already costs up to half a bf16
  ulp, 2^-8 of the value, which for outputs 10 or more times the RMS is above
  the bound by itself; for a bf16 o the bound applies to the error beyond
  that rounding, element by element (:func:`bf16_excess`), and the plain
  figure is reported beside it (:func:`record`).
"""
from __future__ import annotations

import json
import os

import numpy as np


def as64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().float().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


# The smallest normal fp32 value.  An fp32 result cannot hold a value below it
# to any relative precision, so a tensor whose exact values all lie under
# FP32_TINY / 1e-4 (for instance a gradient that carries a decay factor of
# e^-100 ~ 4e-44) is held to an absolute error of FP32_TINY instead.
FP32_TINY = 2.0 ** -126


def max_rel(x, ref, floor: float = 1e-300) -> float:
    """max |x - ref| / max(max |ref|, floor)."""
    x, ref = as64(x), as64(ref)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), floor))


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


def bf16_rounding_floor(ref) -> float:
    """The largest half bf16 ulp over the reference, relative to its RMS: the
    most a bf16 store of an exact value can be off by at one element."""
    return float(bf16_half_ulp(ref).max() / max(rms(ref), 1e-300))


def record(case: str, **figures):
    """Append one JSON line of parity figures to the file named by the
    GDR2_PARITY_LOG environment variable (nothing when it is unset)."""
    path = os.environ.get("GDR2_PARITY_LOG")
    if not path:
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as f:
        f.write(json.dumps({"case": case, **{k: float(v) for k, v in figures.items()}}) + "\n")
