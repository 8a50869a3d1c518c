"""Python binding of libgdr2: the Gated Delta Rule-2 operator on MI355X.

Argument marshalling only.  Every step of the operator runs in the HIP kernels
of ``libgdr2.so`` (built by :mod:`linear_attention_sequence_gdr_amd.build`);
there is no CPU or PyTorch fallback, and calling in without the library raises
:class:`LibraryMissing`.  PyTorch supplies device memory and the stream.

Functions carry the C names (include/gdr2.h):

* :func:`gdr2_chunk_fwd` -- chunkwise forward over whole (optionally packed)
  sequences, returns ``(o, S_T)``.
* :func:`gdr2_decode_step` -- one token for N sequences, updates ``S`` in place,
  returns ``o``.
* :func:`gdr2_chunk_bwd` -- the backward of :func:`gdr2_chunk_fwd`: fp32
  gradients of every input from dL/do and dL/dS_T.
* :func:`gdr2_chunk_fwd_block` -- the forward from the block's projections:
  fused gate prologue (Eq. 12 decay, sigmoid gates, q/k L2 norm) and grouped
  value heads, returns ``(o, S_T)``.
* :func:`gdr2_norm_gate` -- the block's output epilogue (RMSNorm, then a SiLU
  output gate) over o, returns ``y``.
* :func:`gdr2_decode_step_norm_gate` -- a decode step whose store applies that
  epilogue, returns ``y``.
* :func:`gdr2_chunk_fwd_workspace_bytes`, :func:`gdr2_status_string`,
  :func:`gdr2_last_error`, :func:`gdr2_version`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["gdr2_chunk_fwd", "gdr2_chunk_fwd_noalloc", "gdr2_chunk_bwd", "gdr2_chunk_bwd_workspace_bytes", "gdr2_chunk_fwd_block", "gdr2_decode_step", "gdr2_norm_gate",
           "gdr2_decode_step_norm_gate", "GDR2_PRO_QK_L2NORM", "GDR2_PRO_DECAY", "GDR2_PRO_GATES",
           "gdr2_chunk_fwd_workspace_bytes",
           "gdr2_status_string", "gdr2_last_error", "gdr2_version", "Gdr2Error",
           "LibraryMissing", "library", "library_path", "GDR2_F32", "GDR2_BF16", "EXPORTS"]

GDR2_F32, GDR2_BF16 = 0, 1
STATUS = {0: "GDR2_OK", 1: "GDR2_E_NULL", 2: "GDR2_E_SHAPE", 3: "GDR2_E_DTYPE",
          4: "GDR2_E_ALIGN", 5: "GDR2_E_UNSUPPORTED", 6: "GDR2_E_WORKSPACE", 7: "GDR2_E_LAUNCH"}
EXPORTS = ("gdr2_chunk_fwd_workspace_bytes", "gdr2_chunk_fwd", "gdr2_chunk_fwd_f32_out",
           "gdr2_chunk_fwd_noalloc",
           "gdr2_chunk_fwd_block",
           "gdr2_chunk_bwd_workspace_bytes", "gdr2_chunk_bwd", "gdr2_decode_step",
           "gdr2_norm_gate", "gdr2_decode_step_norm_gate",
           "gdr2_status_string", "gdr2_last_error", "gdr2_version")
NORM_GATE_MAX_GROUP = 8192
GDR2_PRO_QK_L2NORM, GDR2_PRO_DECAY, GDR2_PRO_GATES = 1, 2, 4

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libgdr2.so")
_lib = None


class LibraryMissing(RuntimeError):
    pass


class Gdr2Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.name = STATUS.get(status, str(status))


def library():
    """Load libgdr2.so (once) and declare the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise LibraryMissing(
                f"{library_path} is not built; run `python -m linear_attention_sequence_gdr_amd.build`")
        lib = ctypes.CDLL(library_path)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.gdr2_chunk_fwd_workspace_bytes.argtypes = [i32] * 7
        lib.gdr2_chunk_fwd_workspace_bytes.restype = sz
        lib.gdr2_chunk_fwd.argtypes = [vp] * 10 + [i32] * 6 + [i32, i32, vp, sz, vp]
        lib.gdr2_chunk_fwd.restype = i32
        lib.gdr2_chunk_fwd_f32_out.argtypes = lib.gdr2_chunk_fwd.argtypes
        lib.gdr2_chunk_fwd_f32_out.restype = i32
        lib.gdr2_chunk_fwd_noalloc.argtypes = [vp] * 10 + [i32] * 6 + [i32, i32, vp]
        lib.gdr2_chunk_fwd_noalloc.restype = i32
        lib.gdr2_decode_step.argtypes = [vp] * 8 + [i32] * 6 + [vp]
        lib.gdr2_decode_step.restype = i32
        f32, i64 = ctypes.c_float, ctypes.c_longlong
        lib.gdr2_norm_gate.argtypes = [vp] * 4 + [i64, i32, i32, f32, i32, vp]
        lib.gdr2_norm_gate.restype = i32
        lib.gdr2_decode_step_norm_gate.argtypes = [vp] * 9 + [f32, vp] + [i32] * 6 + [vp]
        lib.gdr2_decode_step_norm_gate.restype = i32
        lib.gdr2_chunk_fwd_block.argtypes = [vp] * 8 + [ctypes.c_uint, f32, f32] + [vp] * 4 + \
            [i32] * 7 + [i32, vp, sz, vp]
        lib.gdr2_chunk_fwd_block.restype = i32
        lib.gdr2_chunk_bwd_workspace_bytes.argtypes = [i32] * 6
        lib.gdr2_chunk_bwd_workspace_bytes.restype = sz
        lib.gdr2_chunk_bwd.argtypes = [vp] * 17 + [i32] * 6 + [i32, i32, vp, sz, vp]
        lib.gdr2_chunk_bwd.restype = i32
        lib.gdr2_status_string.argtypes = [i32]
        lib.gdr2_status_string.restype = ctypes.c_char_p
        lib.gdr2_last_error.argtypes = []
        lib.gdr2_last_error.restype = ctypes.c_char_p
        lib.gdr2_version.argtypes = []
        lib.gdr2_version.restype = i32
        _lib = lib
    return _lib


def gdr2_status_string(status: int) -> str:
    return library().gdr2_status_string(int(status)).decode()


def gdr2_last_error() -> str:
    return library().gdr2_last_error().decode()


def gdr2_version() -> int:
    return int(library().gdr2_version())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDR2_BF16
    if t.dtype == torch.float32:
        return GDR2_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor], name: str, device) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _device(x: torch.Tensor, name: str):
    """The device of the leading tensor of a call, which must be a GPU tensor
    (checked before any stream or device query)."""
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    return x.device


def _torch_stream(stream, device):
    """The stream the kernels are enqueued on, as a torch stream: torch's current
    stream on ``device`` when ``stream`` is None, a torch stream as given, or a
    raw hipStream_t handle wrapped as an external stream.  Every call makes it
    current while it allocates its outputs and workspace (and fills any zeros),
    so those tensors belong to that stream: the caching allocator hands their
    memory to later work only in stream order after the kernels that use it."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream(s) -> int:
    return int(s.cuda_stream)


def _check(status: int):
    if status != 0:
        raise Gdr2Error(status, gdr2_last_error())


def gdr2_chunk_fwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, num_seqs: int,
                                   in_dtype: int) -> int:
    return int(library().gdr2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, num_seqs, in_dtype))


def gdr2_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                   b: torch.Tensor, w: torch.Tensor, S0: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, *, o: Optional[torch.Tensor] = None,
                   S_T: Optional[torch.Tensor] = None, want_state: bool = True,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   o_dtype: Optional[torch.dtype] = None):
    """Chunkwise forward.  q, k, log_alpha, b: [B, T, H, dk]; v, w: [B, T, H, dv];
    S0: fp32 [N, H, dk, dv] or None; cu_seqlens: int32 [N+1] (B == 1) or None.
    ``o``/``S_T``/``workspace`` may be passed to avoid allocation.  ``o`` has
    q's dtype by default; an fp32 ``o`` (or ``o_dtype=torch.float32``) with
    bf16 inputs calls gdr2_chunk_fwd_f32_out.  Returns ``(o, S_T)`` (S_T is
    None when ``want_state`` is False and none is given)."""
    lib = library()
    dev = _device(q, "q")
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        return _chunk_fwd(lib, dev, s, q, k, v, log_alpha, b, w, S0, cu_seqlens, o, S_T, want_state,
                          workspace, o_dtype)


def _chunk_fwd(lib, dev, s, q, k, v, log_alpha, b, w, S0, cu_seqlens, o, S_T, want_state, workspace,
               o_dtype):
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    in_dt = _dtype_code(q)
    N = Bsz if cu_seqlens is None else cu_seqlens.numel() - 1
    if o_dtype is None:
        o_dtype = q.dtype if o is None else o.dtype
    if o_dtype not in (q.dtype, torch.float32):
        raise TypeError(f"o_dtype must be {q.dtype} or torch.float32, got {o_dtype}")
    if o is None:
        o = torch.empty((Bsz, T, H, dv), dtype=o_dtype, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    ws_bytes = gdr2_chunk_fwd_workspace_bytes(Bsz, T, H, dk, dv,
                                              N if cu_seqlens is not None else 0, in_dt)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    for name, t, want in (("k", k, q.dtype), ("v", v, q.dtype), ("b", b, q.dtype), ("w", w, q.dtype),
                          ("o", o, o_dtype)):
        if t.dtype != want:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {want}")
    for name, t in (("k", k), ("log_alpha", log_alpha), ("b", b)):
        if tuple(t.shape) != (Bsz, T, H, dk):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(Bsz, T, H, dk)}")
    for name, t in (("w", w), ("o", o)):
        if tuple(t.shape) != (Bsz, T, H, dv):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(Bsz, T, H, dv)}")
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv)):
            raise ValueError(f"{name} must be fp32 {(N, H, dk, dv)}")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    entry = lib.gdr2_chunk_fwd if o_dtype == q.dtype else lib.gdr2_chunk_fwd_f32_out
    st = entry(
        _ptr(q, "q", dev), _ptr(k, "k", dev), _ptr(v, "v", dev), _ptr(log_alpha, "log_alpha", dev),
        _ptr(b, "b", dev), _ptr(w, "w", dev), _ptr(S0, "S0", dev), _ptr(o, "o", dev),
        _ptr(S_T, "S_T", dev), _ptr(cu_seqlens, "cu_seqlens", dev), N if cu_seqlens is not None else 0,
        Bsz, T, H, dk, dv, in_dt, _dtype_code(log_alpha), _ptr(workspace, "workspace", dev),
        ws_bytes, _stream(s))
    _check(st)
    return o, S_T


NOALLOC_SCRATCH_BYTES = 256 << 20


def gdr2_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                           b: torch.Tensor, w: torch.Tensor, S0: Optional[torch.Tensor],
                           cu_seqlens: Optional[torch.Tensor], o: torch.Tensor,
                           S_T: Optional[torch.Tensor], stream=None):
    """gdr2_chunk_fwd on the library's static scratch: the caller passes every
    output (o in q's dtype, S_T fp32 or None) and nothing is allocated, by
    this binding or the library.  Returns ``(o, S_T)``."""
    lib = library()
    dev = _device(q, "q")
    s = _torch_stream(stream, dev)
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    N = Bsz if cu_seqlens is None else cu_seqlens.numel() - 1
    for name, t in (("k", k), ("v", v), ("b", b), ("w", w), ("o", o)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    for name, t, shp in (("k", k, (Bsz, T, H, dk)), ("log_alpha", log_alpha, (Bsz, T, H, dk)),
                         ("b", b, (Bsz, T, H, dk)), ("v", v, (Bsz, T, H, dv)), ("w", w, (Bsz, T, H, dv)),
                         ("o", o, (Bsz, T, H, dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv)):
            raise ValueError(f"{name} must be fp32 {(N, H, dk, dv)}")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    st = lib.gdr2_chunk_fwd_noalloc(
        _ptr(q, "q", dev), _ptr(k, "k", dev), _ptr(v, "v", dev), _ptr(log_alpha, "log_alpha", dev),
        _ptr(b, "b", dev), _ptr(w, "w", dev), _ptr(S0, "S0", dev), _ptr(o, "o", dev),
        _ptr(S_T, "S_T", dev), _ptr(cu_seqlens, "cu_seqlens", dev), N if cu_seqlens is not None else 0,
        Bsz, T, H, dk, dv, _dtype_code(q), _dtype_code(log_alpha), _stream(s))
    _check(st)
    return o, S_T


def gdr2_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                     b: torch.Tensor, w: torch.Tensor, S: torch.Tensor, *,
                     o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step.  q, k, log_alpha, b: [N, H, dk]; v, w: [N, H, dv];
    S: fp32 [N, H, dk, dv] updated in place.  Returns o [N, H, dv]."""
    lib = library()
    dev = _device(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    s = _torch_stream(stream, dev)
    if o is None:
        with torch.cuda.stream(s):
            o = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    for name, t, shp in (("k", k, (N, H, dk)), ("log_alpha", log_alpha, (N, H, dk)),
                         ("b", b, (N, H, dk)), ("v", v, (N, H, dv)), ("w", w, (N, H, dv)),
                         ("o", o, (N, H, dv)), ("S", S, (N, H, dk, dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    if S.dtype != torch.float32:
        raise TypeError("S must be fp32")
    st = lib.gdr2_decode_step(
        _ptr(q, "q", dev), _ptr(k, "k", dev), _ptr(v, "v", dev), _ptr(log_alpha, "log_alpha", dev),
        _ptr(b, "b", dev), _ptr(w, "w", dev), _ptr(S, "S", dev), _ptr(o, "o", dev),
        N, H, dk, dv, _dtype_code(q), _dtype_code(log_alpha), _stream(s))
    _check(st)
    return o


def gdr2_norm_gate(o: torch.Tensor, z: torch.Tensor, weight: Optional[torch.Tensor] = None,
                   eps: float = 1e-6, group: Optional[int] = None, *,
                   y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Output epilogue y = o / sqrt(mean(o^2) + eps) * weight * silu(z), the
    mean taken over groups of ``group`` channels of the last axis (default: the
    whole last axis).  o, z (and y): one shape, bf16 or fp32; weight: fp32
    [o.shape[-1]] or None.  ``y`` may be ``o`` or ``z`` (in place)."""
    lib = library()
    dev = _device(o, "o")
    d = o.shape[-1]
    group = d if group is None else int(group)
    if z.shape != o.shape or z.dtype != o.dtype:
        raise ValueError(f"z must match o ({tuple(o.shape)}, {o.dtype}), got {tuple(z.shape)}, {z.dtype}")
    s = _torch_stream(stream, dev)
    if y is None:
        with torch.cuda.stream(s):
            y = torch.empty_like(o)
    if y.shape != o.shape or y.dtype != o.dtype:
        raise ValueError("y must match o in shape and dtype")
    if weight is not None and (weight.dtype != torch.float32 or tuple(weight.shape) != (d,)):
        raise ValueError(f"weight must be fp32 [{d}]")
    rows = o.numel() // d if d else 0
    st = lib.gdr2_norm_gate(_ptr(o, "o", dev), _ptr(z, "z", dev), _ptr(weight, "weight", dev),
                            _ptr(y, "y", dev), rows, d, group, float(eps), _dtype_code(o),
                            _stream(s))
    _check(st)
    return y


def gdr2_decode_step_norm_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               log_alpha: torch.Tensor, b: torch.Tensor, w: torch.Tensor,
                               S: torch.Tensor, z: torch.Tensor,
                               norm_weight: Optional[torch.Tensor] = None, eps: float = 1e-6, *,
                               y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step (S updated in place) whose output is the epilogue
    RMSNorm(o) * norm_weight * silu(z) over each head's dv channels.  z: [N, H,
    dv] in q's dtype; norm_weight: fp32 [dv] or None.  Returns y [N, H, dv]."""
    lib = library()
    dev = _device(q, "q")
    N, H, dk = q.shape
    dv = v.shape[-1]
    s = _torch_stream(stream, dev)
    if y is None:
        with torch.cuda.stream(s):
            y = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    for name, t, shp in (("k", k, (N, H, dk)), ("log_alpha", log_alpha, (N, H, dk)),
                         ("b", b, (N, H, dk)), ("v", v, (N, H, dv)), ("w", w, (N, H, dv)),
                         ("z", z, (N, H, dv)), ("y", y, (N, H, dv)), ("S", S, (N, H, dk, dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    for name, t in (("z", z), ("y", y)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    if S.dtype != torch.float32:
        raise TypeError("S must be fp32")
    if norm_weight is not None and (norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (dv,)):
        raise ValueError(f"norm_weight must be fp32 [{dv}]")
    st = lib.gdr2_decode_step_norm_gate(
        _ptr(q, "q", dev), _ptr(k, "k", dev), _ptr(v, "v", dev), _ptr(log_alpha, "log_alpha", dev),
        _ptr(b, "b", dev), _ptr(w, "w", dev), _ptr(S, "S", dev), _ptr(z, "z", dev),
        _ptr(norm_weight, "norm_weight", dev), float(eps), _ptr(y, "y", dev),
        N, H, dk, dv, _dtype_code(q), _dtype_code(log_alpha), _stream(s))
    _check(st)
    return y


def gdr2_chunk_fwd_block(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, f: torch.Tensor,
                         b: torch.Tensor, w: torch.Tensor, decay_a: Optional[torch.Tensor] = None,
                         decay_bias: Optional[torch.Tensor] = None, *,
                         flags: int = GDR2_PRO_QK_L2NORM | GDR2_PRO_DECAY | GDR2_PRO_GATES,
                         b_scale: float = 1.0, qk_eps: float = 1e-6,
                         S0: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                         o: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                         want_state: bool = True, workspace: Optional[torch.Tensor] = None,
                         stream=None):
    """Forward from the block's projections.  q, k, f, b: [B, T, H, dk]; v, w:
    [B, T, Hv, dv] (Hv a multiple of H); all bf16 except f (bf16 or fp32).
    ``flags`` selects the prologue steps (GDR2_PRO_*): f is W_f x under
    GDR2_PRO_DECAY (decay_a, decay_bias: fp32 [H, dk]), b and w are W_b x and
    W_w x under GDR2_PRO_GATES, q and k are L2-normalised under
    GDR2_PRO_QK_L2NORM.  Returns ``(o [B, T, Hv, dv], S_T [N, Hv, dk, dv])``."""
    lib = library()
    dev = _device(q, "q")
    if q.dtype != torch.bfloat16:
        raise TypeError("gdr2_chunk_fwd_block takes bf16 q, k, v, b, w")
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        return _chunk_fwd_block(lib, dev, s, q, k, v, f, b, w, decay_a, decay_bias, flags, b_scale,
                                qk_eps, S0, cu_seqlens, o, S_T, want_state, workspace)


def _chunk_fwd_block(lib, dev, s, q, k, v, f, b, w, decay_a, decay_bias, flags, b_scale, qk_eps, S0,
                     cu_seqlens, o, S_T, want_state, workspace):
    Bsz, T, H, dk = q.shape
    Hv, dv = v.shape[-2], v.shape[-1]
    N = Bsz if cu_seqlens is None else cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((Bsz, T, Hv, dv), dtype=torch.bfloat16, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=dev)
    ns = N if cu_seqlens is not None else 0
    ws_bytes = gdr2_chunk_fwd_workspace_bytes(Bsz, T, Hv, dk, dv, ns, GDR2_BF16)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    for name, t, shp in (("k", k, (Bsz, T, H, dk)), ("f", f, (Bsz, T, H, dk)), ("b", b, (Bsz, T, H, dk)),
                         ("v", v, (Bsz, T, Hv, dv)), ("w", w, (Bsz, T, Hv, dv)), ("o", o, (Bsz, T, Hv, dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
        if name != "f" and t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bf16")
    for name, t in (("decay_a", decay_a), ("decay_bias", decay_bias)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (H, dk)):
            raise ValueError(f"{name} must be fp32 {(H, dk)}")
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, Hv, dk, dv)):
            raise ValueError(f"{name} must be fp32 {(N, Hv, dk, dv)}")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    st = lib.gdr2_chunk_fwd_block(
        _ptr(q, "q", dev), _ptr(k, "k", dev), _ptr(v, "v", dev), _ptr(f, "f", dev), _ptr(b, "b", dev),
        _ptr(w, "w", dev), _ptr(decay_a, "decay_a", dev), _ptr(decay_bias, "decay_bias", dev),
        int(flags), float(b_scale), float(qk_eps), _ptr(S0, "S0", dev), _ptr(o, "o", dev),
        _ptr(S_T, "S_T", dev), _ptr(cu_seqlens, "cu_seqlens", dev), ns, Bsz, T, H, Hv, dk, dv,
        _dtype_code(f), _ptr(workspace, "workspace", dev), ws_bytes, _stream(s))
    _check(st)
    return o, S_T


def gdr2_chunk_bwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, num_seqs: int) -> int:
    return int(library().gdr2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs))


def gdr2_chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                   b: torch.Tensor, w: torch.Tensor, dO: torch.Tensor,
                   S0: Optional[torch.Tensor] = None, dS_T: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, *, want_dS0: bool = True,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Backward of :func:`gdr2_chunk_fwd`.  Inputs as for the forward; dO:
    dL/do [B, T, H, dv] in q's dtype; dS_T: fp32 [N, H, dk, dv] or None.
    Returns a dict of fp32 gradients dq, dk, dlog_alpha, db [B, T, H, dk],
    dv, dw [B, T, H, dv] and dS0 [N, H, dk, dv] (None unless ``want_dS0``)."""
    lib = library()
    dev = _device(q, "q")
    s = _torch_stream(stream, dev)
    with torch.cuda.stream(s):
        return _chunk_bwd(lib, dev, s, q, k, v, log_alpha, b, w, dO, S0, dS_T, cu_seqlens, want_dS0,
                          workspace)


def _chunk_bwd(lib, dev, s, q, k, v, log_alpha, b, w, dO, S0, dS_T, cu_seqlens, want_dS0, workspace):
    Bsz, T, H, dk = q.shape
    dv = v.shape[-1]
    N = Bsz if cu_seqlens is None else cu_seqlens.numel() - 1
    ns = N if cu_seqlens is not None else 0
    for name, t, shp in (("k", k, (Bsz, T, H, dk)), ("log_alpha", log_alpha, (Bsz, T, H, dk)),
                         ("b", b, (Bsz, T, H, dk)), ("v", v, (Bsz, T, H, dv)), ("w", w, (Bsz, T, H, dv)),
                         ("dO", dO, (Bsz, T, H, dv))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    for name, t in (("k", k), ("v", v), ("b", b), ("w", w), ("dO", dO)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv)):
            raise ValueError(f"{name} must be fp32 {(N, H, dk, dv)}")
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    f32 = torch.float32
    # every row is written unless packed sequences leave rows outside [cu[0], cu[N])
    alloc = torch.empty if cu_seqlens is None else torch.zeros
    g = {n: alloc((Bsz, T, H, dk), dtype=f32, device=dev) for n in ("dq", "dk", "dlog_alpha", "db")}
    g.update({n: alloc((Bsz, T, H, dv), dtype=f32, device=dev) for n in ("dv", "dw")})
    g["dS0"] = torch.empty((N, H, dk, dv), dtype=f32, device=dev) if want_dS0 else None
    ws_bytes = gdr2_chunk_bwd_workspace_bytes(Bsz, T, H, dk, dv, ns)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.gdr2_chunk_bwd(
        _ptr(q, "q", dev), _ptr(k, "k", dev), _ptr(v, "v", dev), _ptr(log_alpha, "log_alpha", dev),
        _ptr(b, "b", dev), _ptr(w, "w", dev), _ptr(S0, "S0", dev), _ptr(dO, "dO", dev),
        _ptr(dS_T, "dS_T", dev), _ptr(g["dq"], "dq", dev), _ptr(g["dk"], "dk", dev),
        _ptr(g["dv"], "dv", dev), _ptr(g["dlog_alpha"], "dlog_alpha", dev), _ptr(g["db"], "db", dev),
        _ptr(g["dw"], "dw", dev), _ptr(g["dS0"], "dS0", dev), _ptr(cu_seqlens, "cu_seqlens", dev),
        ns, Bsz, T, H, dk, dv, _dtype_code(q), _dtype_code(log_alpha), _ptr(workspace, "workspace", dev),
        ws_bytes, _stream(s))
    _check(st)
    return g
