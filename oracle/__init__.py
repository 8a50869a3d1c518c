"""fp64 CPU oracle for the Gated Delta Rule-2 operator (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The GPU library never loads it, and it shares no code
with the GPU library.

* :func:`fwd` / :func:`decode` -- the token-by-token recurrence in fp64
  (``gdr2_oracle.c``; Gated DeltaNet-2 pages, Steps 1-5 and Eq. 10).
* :func:`bwd` -- reverse-mode differentiation of that recurrence in fp64
  (``gdr2_oracle_bwd.c``; the pages' gate-aware backward flow): dq, dk, dv,
  dlog_alpha, db, dw and dS0 from dL/do and dL/dS_T.
* :mod:`oracle.chunk_ref` -- the pages' chunkwise WY algorithm in fp64 numpy,
  used to pin the recurrence (the two must agree to rounding).
* :mod:`oracle.epilogue` -- the block's output epilogue, RMSNorm then a SiLU
  output gate, in fp64 numpy (pages, "Big-Picture Architecture" item 6).
* :mod:`oracle.prologue` -- the gate prologue (Eq. 12 log-decay, Eq. 11
  sigmoid gates, q/k L2 norm) and grouped value heads, in fp64 numpy, producing
  the operator's inputs for :func:`fwd`.

Inputs are the *stored* tensors (bf16 or fp32), converted exactly to fp64, so
the comparison measures the kernel's arithmetic and not input quantisation.
Parity status of every function here is recorded in the test modules that pin
it; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libgdr2_oracle.so")
_BWD_SRC = os.path.join(_HERE, "gdr2_oracle_bwd.c")
_BWD_LIB_PATH = os.path.join(_HERE, "_build", "libgdr2_oracle_bwd.so")
_lib = None
_bwd_lib = None


def _gcc(src: str, out: str):
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                           "-Wall", "-Werror", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)


def build(force: bool = True) -> str:
    """Compile the C oracle (forward and backward libraries) with gcc (-O2,
    OpenMP) into oracle/_build."""
    for src, out in ((_SRC, _LIB_PATH), (_BWD_SRC, _BWD_LIB_PATH)):
        if force or not os.path.exists(out):
            _gcc(src, out)
    return _LIB_PATH


def load_library(path: str):
    """Load a compiled oracle library (the default build, or a test-built
    variant) and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gdr2_oracle_fwd.argtypes = [dp] * 6 + [ctypes.c_void_p, dp, ctypes.c_void_p,
                                               ctypes.POINTER(ctypes.c_longlong)] + \
        [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_int]
    lib.gdr2_oracle_fwd.restype = ctypes.c_int
    lib.gdr2_oracle_decode.argtypes = [dp] * 8 + [ctypes.c_int] * 5
    lib.gdr2_oracle_decode.restype = ctypes.c_int
    lib.gdr2_oracle_max_threads.restype = ctypes.c_int
    return lib


def load_bwd_library(path: str):
    """Load a compiled backward oracle library and declare its C signature."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gdr2_oracle_bwd.argtypes = [dp] * 6 + [ctypes.c_void_p, dp, ctypes.c_void_p] + [dp] * 6 + \
        [ctypes.c_void_p, ctypes.POINTER(ctypes.c_longlong)] + [ctypes.c_int] * 4 + \
        [ctypes.c_void_p, ctypes.c_int]
    lib.gdr2_oracle_bwd.restype = ctypes.c_int
    return lib


def _load_bwd():
    global _bwd_lib
    if _bwd_lib is None:
        if not os.path.exists(_BWD_LIB_PATH) or os.path.getmtime(_BWD_LIB_PATH) < os.path.getmtime(_BWD_SRC):
            _gcc(_BWD_SRC, _BWD_LIB_PATH)
        _bwd_lib = load_bwd_library(_BWD_LIB_PATH)
    return _bwd_lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def f64(x) -> np.ndarray:
    """Exact conversion of a stored tensor (torch bf16/fp32, or numpy) to a
    C-contiguous fp64 array."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().gdr2_oracle_max_threads())


def fwd(q, k, v, g, b, w, S0=None, cu_seqlens=None, mask=None, nthreads: int = 0, lib=None):
    """Token-by-token fp64 forward.

    q, k, g, b: [B, T, H, dk]; v, w: [B, T, H, dv] (torch or numpy, any float
    dtype; converted exactly).  ``cu_seqlens`` packs sequences along the
    flattened B*T token axis (None: each batch row is one sequence).  ``S0`` is
    [N, H, dk, dv] or None (zeros).  ``mask`` ([N, H] bool) restricts the work
    to selected (sequence, head) pairs.  Returns (o [B, T, H, dv], S_T
    [N, H, dk, dv]) in fp64.
    """
    q, k, v, g, b, w = (f64(x) for x in (q, k, v, g, b, w))
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(Bsz + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.size - 1
    o = np.zeros((Bsz, T, H, dv), dtype=np.float64)
    ST = np.zeros((N, H, dk, dv), dtype=np.float64)
    s0 = None if S0 is None else f64(S0)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    m = None
    if mask is not None:
        m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(N * H))
    rc = (lib or _load()).gdr2_oracle_fwd(
        _p(q), _p(k), _p(v), _p(g), _p(b), _p(w),
        None if s0 is None else s0.ctypes.data_as(ctypes.c_void_p), _p(o),
        ST.ctypes.data_as(ctypes.c_void_p),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)), N, H, dk, dv,
        None if m is None else m.ctypes.data_as(ctypes.c_void_p), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle forward rejected its arguments")
    return o, ST


def decode(q, k, v, g, b, w, S, nthreads: int = 0, lib=None, inplace: bool = False):
    """One fp64 decode step.  Inputs [N, H, d]; S [N, H, dk, dv].  Returns
    (o [N, H, dv], S_new).  S is not modified unless ``inplace``, which needs a
    C-contiguous float64 numpy S and updates it (S_new is then S itself)."""
    q, k, v, g, b, w = (f64(x) for x in (q, k, v, g, b, w))
    if inplace:
        if not (isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous):
            raise TypeError("inplace decode needs a C-contiguous float64 numpy state")
    else:
        S = f64(S).copy()
    N, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = (lib or _load()).gdr2_oracle_decode(_p(q), _p(k), _p(v), _p(g), _p(b), _p(w), _p(S), _p(o),
                                    N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle decode rejected its arguments")
    return o, S


def bwd(q, k, v, g, b, w, dO, S0=None, dST=None, cu_seqlens=None, mask=None, nthreads: int = 0,
        lib=None):
    """Token-by-token fp64 backward of :func:`fwd`.

    Same layouts as :func:`fwd`; ``dO`` is dL/do [B, T, H, dv] and ``dST``
    dL/dS_T [N, H, dk, dv] (None: zero).  Returns a dict with dq, dk, dg, db
    [B, T, H, dk], dv, dw [B, T, H, dv] and dS0 [N, H, dk, dv] (fp64)."""
    q, k, v, g, b, w, dO = (f64(x) for x in (q, k, v, g, b, w, dO))
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    cu = (np.arange(Bsz + 1, dtype=np.int64) * T if cu_seqlens is None
          else np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64)))
    N = cu.size - 1
    out = {n: np.zeros((Bsz, T, H, dk)) for n in ("dq", "dk", "dg", "db")}
    out.update({n: np.zeros((Bsz, T, H, dv)) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((N, H, dk, dv))
    s0 = None if S0 is None else f64(S0)
    dst = None if dST is None else f64(dST)
    m = None
    if mask is not None:
        m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(N * H))
    vp = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = (lib or _load_bwd()).gdr2_oracle_bwd(
        _p(q), _p(k), _p(v), _p(g), _p(b), _p(w), vp(s0), _p(dO), vp(dst),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dg"]), _p(out["db"]), _p(out["dw"]),
        vp(out["dS0"]), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)), N, H, dk, dv,
        vp(m), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle backward rejected its arguments")
    return out
