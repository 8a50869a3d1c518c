"""Seeded synthetic inputs for the Gated Delta Rule-2 operator.

This module is shared by the tests, the benchmark and the smoke check.  It
draws random tensors with the distributions of the five standard workloads
and holds none of the operator's arithmetic: the recurrence, the chunkwise
algorithm and every error metric live elsewhere.  The value transforms here
(L2 normalisation, sigmoid, softplus) only shape the input distributions the
way the block upstream of the operator would (Gated DeltaNet-2 pages: block
design, q/k L2-normalised per head; gate parameterisation, Eqs. 11-12).

Layout: token tensors are ``[B, T, H, D]`` contiguous (D fastest); the state is
``[N, H, dk, dv]`` fp32.  Draws happen in fp32 on the CPU with
``torch.Generator('cpu').manual_seed(seed)`` in a fixed order, then the values
are cast to the storage dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass
class Workload:
    """One synthetic forward workload (all tensors on the CPU)."""

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    log_alpha: torch.Tensor
    b: torch.Tensor
    w: torch.Tensor
    S0: Optional[torch.Tensor]          # [N, H, dk, dv] fp32 or None (zeros)
    cu_seqlens: Optional[torch.Tensor]  # int32 [N+1] or None (N = B)
    seed: int

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.q.shape[2]

    @property
    def dk(self) -> int:
        return self.q.shape[3]

    @property
    def dv(self) -> int:
        return self.v.shape[3]

    @property
    def num_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1


def _l2n(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def draw_tokens(gen: torch.Generator, B: int, T: int, H: int, dk: int, dv: int,
                dtype: torch.dtype, la_dtype: torch.dtype, decay_shift: float,
                erase_scale: float = 1.0, tie: str = "none"):
    """Draw (q, k, v, log_alpha, b, w) of shape [B, T, H, *].

    q, k ~ N(0, 1) L2-normalised over the key axis; v ~ N(0, 1);
    b = erase_scale * sigmoid(N(0, 1)); w = sigmoid(N(0, 1));
    log_alpha = -softplus(N(0, 1) + decay_shift).

    tie="kda": b and w are one scalar beta = sigmoid(N(0,1)) per (token, head)
    broadcast over their channels.  tie="gdn": additionally log_alpha is one
    scalar per (token, head) broadcast over the key channels.
    """
    f32 = torch.float32
    q = _l2n(torch.randn(B, T, H, dk, generator=gen, dtype=f32))
    k = _l2n(torch.randn(B, T, H, dk, generator=gen, dtype=f32))
    v = torch.randn(B, T, H, dv, generator=gen, dtype=f32)
    if tie == "none":
        b = erase_scale * torch.sigmoid(torch.randn(B, T, H, dk, generator=gen, dtype=f32))
        w = torch.sigmoid(torch.randn(B, T, H, dv, generator=gen, dtype=f32))
        la = -torch.nn.functional.softplus(
            torch.randn(B, T, H, dk, generator=gen, dtype=f32) + decay_shift)
    else:
        beta = torch.sigmoid(torch.randn(B, T, H, 1, generator=gen, dtype=f32))
        b = (erase_scale * beta).expand(B, T, H, dk).contiguous()
        w = beta.expand(B, T, H, dv).contiguous()
        if tie == "gdn":
            la = -torch.nn.functional.softplus(
                torch.randn(B, T, H, 1, generator=gen, dtype=f32) + decay_shift)
            la = la.expand(B, T, H, dk).contiguous()
        else:
            la = -torch.nn.functional.softplus(
                torch.randn(B, T, H, dk, generator=gen, dtype=f32) + decay_shift)
    return (q.to(dtype), k.to(dtype), v.to(dtype), la.to(la_dtype), b.to(dtype), w.to(dtype))


def draw_state(gen: torch.Generator, N: int, H: int, dk: int, dv: int, std: float = 0.1):
    return (std * torch.randn(N, H, dk, dv, generator=gen, dtype=torch.float32)).contiguous()


def make_forward(B: int, T: int, H: int, dk: int, dv: int, *, dtype=torch.bfloat16,
                 la_dtype=None, decay_shift: float = -2.0, erase_scale: float = 1.0,
                 s0_std: float = 0.0, seqlens=None, tie: str = "none", seed: int = 0,
                 name: str = "custom") -> Workload:
    """A general seeded forward workload.  ``seqlens`` (a list) packs
    variable-length sequences into one row (B must be 1, T = sum)."""
    la_dtype = dtype if la_dtype is None else la_dtype
    gen = torch.Generator("cpu").manual_seed(seed)
    cu = None
    if seqlens is not None:
        assert B == 1 and sum(seqlens) == T
        cu = torch.zeros(len(seqlens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0).to(torch.int32)
    q, k, v, la, b, w = draw_tokens(gen, B, T, H, dk, dv, dtype, la_dtype, decay_shift,
                                    erase_scale, tie)
    N = B if cu is None else cu.numel() - 1
    S0 = draw_state(gen, N, H, dk, dv, s0_std) if s0_std > 0 else None
    return Workload(name, q, k, v, la, b, w, S0, cu, seed)


def varlen_lengths(seed: int, num_seqs: int = 64, max_len: int = 8192):
    """Sequence lengths drawn uniformly from [1, max_len] with their own seed."""
    gen = torch.Generator("cpu").manual_seed(seed)
    return torch.randint(1, max_len + 1, (num_seqs,), generator=gen).tolist()


def config(index: int, *, variant: str = "none") -> Workload:
    """The five standard workloads.

    0: tiny fp32 forward, B1 T256 H2 d32, decay shift 0 (variant "kda"/"gdn"
       gives the tied-gate and scalar-decay collapses).
    1: training-shape forward, B4 T4096 H16 d128, bf16, decay shift -2, S0=0.
    2: decode (use :func:`decode_state` / :func:`decode_step_inputs`).
    3: long context, B1 T32768 H16 d128, bf16, b in [0,2], decay shift -4,
       S0 ~ N(0, 0.1).
    4: packed varlen, 64 sequences of U[1, 8192] tokens, H16 d128, bf16,
       decay shift -2, per-sequence S0 ~ N(0, 0.1).
    """
    seed = 1000 + index
    if index == 0:
        return make_forward(1, 256, 2, 32, 32, dtype=torch.float32, decay_shift=0.0,
                            tie=variant, seed=seed, name=f"cfg0-{variant}")
    if index == 1:
        return make_forward(4, 4096, 16, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                            seed=seed, name="cfg1")
    if index == 3:
        return make_forward(1, 32768, 16, 128, 128, dtype=torch.bfloat16, decay_shift=-4.0,
                            erase_scale=2.0, s0_std=0.1, seed=seed, name="cfg3")
    if index == 4:
        lens = varlen_lengths(seed + 7)
        return make_forward(1, sum(lens), 16, 128, 128, dtype=torch.bfloat16,
                            decay_shift=-2.0, s0_std=0.1, seqlens=lens, seed=seed,
                            name="cfg4")
    raise ValueError(f"no forward workload for config {index}")


def packed_long(seed: int = 1010) -> Workload:
    """One 32,768-token sequence among 63 short ones of U[1, 512] tokens (the
    long one at index 20), packed by cu_seqlens, H16 dk=dv=128 bf16, gates as
    in config 1, per-sequence S0 ~ N(0, 0.1)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lens = torch.randint(1, 513, (64,), generator=gen).tolist()
    lens[20] = 32768
    return make_forward(1, sum(lens), 16, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=seed, name="packed-long")


# ---- decode (config 2) -------------------------------------------------------------

DECODE_N, DECODE_H, DECODE_D, DECODE_STEPS = 256, 16, 128, 512


def decode_state(N: int = DECODE_N, H: int = DECODE_H, dk: int = DECODE_D,
                 dv: int = DECODE_D, seed: int = 1002) -> torch.Tensor:
    gen = torch.Generator("cpu").manual_seed(seed)
    return draw_state(gen, N, H, dk, dv, 0.1)


def decode_step_inputs(step: int, N: int = DECODE_N, H: int = DECODE_H, dk: int = DECODE_D,
                       dv: int = DECODE_D, dtype=torch.float32, seed: int = 1002):
    """Per-token inputs of decode step ``step``, shaped [N, H, D] (drawn as the
    tiny fp32 forward: decay shift 0)."""
    gen = torch.Generator("cpu").manual_seed(seed * 100003 + step + 1)
    q, k, v, la, b, w = draw_tokens(gen, N, 1, H, dk, dv, dtype, dtype, 0.0)
    return tuple(x[:, 0].contiguous() for x in (q, k, v, la, b, w))


# ---- output epilogue ---------------------------------------------------------------

def epilogue_inputs(shape, *, dtype=torch.bfloat16, seed: int = 1005, weight: bool = True):
    """Inputs of the output epilogue (RMSNorm, then a SiLU output gate): o of
    ``shape`` whose rows (last axis) carry scales spread over e^-1..e^1 around
    N(0, 1) values, the gate pre-activation z ~ N(0, 1.5^2), and a per-channel
    fp32 weight 1 + N(0, 0.1^2) over the last axis (None when ``weight`` is
    False)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    f32 = torch.float32
    o = torch.randn(*shape, generator=gen, dtype=f32)
    o = o * torch.exp(torch.rand(*shape[:-1], 1, generator=gen, dtype=f32) * 2 - 1)
    z = 1.5 * torch.randn(*shape, generator=gen, dtype=f32)
    wt = 1 + 0.1 * torch.randn(shape[-1], generator=gen, dtype=f32) if weight else None
    return o.to(dtype).contiguous(), z.to(dtype).contiguous(), wt


# ---- block inputs: projections before the gate prologue ------------------------------

@dataclasses.dataclass
class BlockWorkload:
    """Inputs of the forward from the block's projections (all on the CPU).
    q, k, f, b: [B, T, H, dk]; v, w: [B, T, Hv, dv]; a, delta: fp32 [H, dk]."""

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    f: torch.Tensor
    b: torch.Tensor
    w: torch.Tensor
    a: torch.Tensor
    delta: torch.Tensor
    S0: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    seed: int


def make_block(B: int, T: int, H: int, Hv: int, dk: int, dv: int, *, f_dtype=torch.bfloat16,
               s0_std: float = 0.0, seqlens=None, seed: int = 0, name: str = "block") -> BlockWorkload:
    """Raw q, k ~ N(0, 1) (not normalised), v ~ N(0, 1), pre-activations f, b,
    w ~ N(0, 1); a = log U[1, 16] and delta = softplus^-1(dt) with dt
    log-uniform in [1e-3, 1e-1] per (key head, channel), so that the per-token
    decay -exp(a) * softplus(f + delta) lies mostly in [-0.3, -0.02]."""
    gen = torch.Generator("cpu").manual_seed(seed)
    f32 = torch.float32
    cu = None
    if seqlens is not None:
        assert B == 1 and sum(seqlens) == T
        cu = torch.zeros(len(seqlens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(seqlens, dtype=torch.int64), 0).to(torch.int32)
    q = torch.randn(B, T, H, dk, generator=gen, dtype=f32)
    k = torch.randn(B, T, H, dk, generator=gen, dtype=f32)
    v = torch.randn(B, T, Hv, dv, generator=gen, dtype=f32)
    f = torch.randn(B, T, H, dk, generator=gen, dtype=f32)
    b = torch.randn(B, T, H, dk, generator=gen, dtype=f32)
    w = torch.randn(B, T, Hv, dv, generator=gen, dtype=f32)
    a = torch.log(1 + 15 * torch.rand(H, dk, generator=gen, dtype=f32))
    dt = torch.exp(torch.log(torch.tensor(1e-3)) + torch.rand(H, dk, generator=gen, dtype=f32)
                   * (torch.log(torch.tensor(1e-1)) - torch.log(torch.tensor(1e-3))))
    delta = torch.log(torch.expm1(dt))
    N = B if cu is None else cu.numel() - 1
    S0 = draw_state(gen, N, Hv, dk, dv, s0_std) if s0_std > 0 else None
    bf = torch.bfloat16
    return BlockWorkload(name, q.to(bf), k.to(bf), v.to(bf), f.to(f_dtype), b.to(bf), w.to(bf),
                         a.contiguous(), delta.contiguous(), S0, cu, seed)


# ---- backward: cotangents ------------------------------------------------------------

def cotangents(wl: Workload, *, seed: int = 7, ds_std: float = 0.1):
    """dL/do ~ N(0, 1) in the workload's storage dtype, shaped like o, and
    dL/dS_T ~ N(0, ds_std^2) fp32 per sequence."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dO = torch.randn(wl.B, wl.T, wl.H, wl.dv, generator=gen, dtype=torch.float32).to(wl.q.dtype)
    dST = ds_std * torch.randn(wl.num_seqs, wl.H, wl.dk, wl.dv, generator=gen, dtype=torch.float32)
    return dO.contiguous(), dST.contiguous()
