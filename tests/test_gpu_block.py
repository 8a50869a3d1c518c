"""Forward from the block's projections on the GPU (fused gate prologue and
grouped value heads) against the fp64 oracle, through the C ABI (needs an
MI355X).

The oracle applies the prologue in fp64 to the same stored pre-activations
(oracle.prologue.block_inputs) and runs the token-by-token recurrence on the
result, with the key-side tensors repeated across each value-head group.
Tolerance: that of the bf16 forward, max-abs error over the reference RMS
<= 2e-2 on S_T and on o beyond o's own bf16 rounding (tests/metrics.py).
"""
import numpy as np
import pytest
import torch

import gdr2_inputs as I
import oracle
from oracle import prologue as P
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = 2e-2
ALL = 7


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def run_block(wl, flags=ALL, b_scale=1.0, qk_eps=1e-6, **kw):
    dev = lambda x: None if x is None else x.cuda()
    o, ST = G().gdr2_chunk_fwd_block(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.f), dev(wl.b), dev(wl.w),
                                     dev(wl.a), dev(wl.delta), flags=flags, b_scale=b_scale,
                                     qk_eps=qk_eps, S0=dev(wl.S0), cu_seqlens=dev(wl.cu_seqlens), **kw)
    torch.cuda.synchronize()
    return o.cpu(), None if ST is None else ST.cpu()


def oracle_block(wl, flags=ALL, b_scale=1.0, qk_eps=1e-6, mask=None):
    ins = P.block_inputs(wl.q, wl.k, wl.v, wl.f, wl.b, wl.w, wl.a, wl.delta, b_scale=b_scale,
                         qk_eps=qk_eps, qk_norm=bool(flags & 1), decay=bool(flags & 2),
                         gates=bool(flags & 4))
    cu = None if wl.cu_seqlens is None else wl.cu_seqlens.numpy()
    return oracle.fwd(*ins, S0=wl.S0, cu_seqlens=cu, mask=mask)


def check(o, ST, ro, rS, what):
    eo, es, plain = M.bf16_excess(o, ro), M.rms_err(ST, rS), M.rms_err(o, ro)
    M.record(what, o_beyond_bf16_rounding=eo, o_plain=plain,
             o_bf16_rounding_floor=M.bf16_rounding_floor(ro), S_T=es)
    assert eo <= TOL and es <= TOL, f"{what}: o excess {eo:.3e} (plain {plain:.3e}), S_T {es:.3e}"


@pytest.mark.parametrize("B,T,H,Hv,dk,dv,fdt,bs", [
    (2, 203, 2, 4, 128, 128, torch.bfloat16, 1.0),
    (2, 203, 2, 2, 128, 128, torch.float32, 2.0),
    (1, 130, 4, 4, 64, 32, torch.bfloat16, 2.0),
    (2, 77, 1, 4, 32, 64, torch.float32, 1.0),
    (1, 64, 2, 8, 128, 64, torch.bfloat16, 1.0),
])
def test_block_all_steps(B, T, H, Hv, dk, dv, fdt, bs):
    wl = I.make_block(B, T, H, Hv, dk, dv, f_dtype=fdt, s0_std=0.1, seed=31 + T + Hv)
    o, ST = run_block(wl, b_scale=bs)
    ro, rS = oracle_block(wl, b_scale=bs)
    check(o, ST, ro, rS, f"B{B} T{T} H{H} Hv{Hv} dk{dk} dv{dv} {fdt} b_scale {bs}")


def test_block_grouped_heads_split_chains():
    """Few long chains: 1 sequence x 4 value heads of 64 chunks takes the split
    state pass (4 segments of 16 chunks per chain, a transfer pass and a scan)
    behind the prologue and the key-head broadcast (2 key heads, groups of 2)."""
    B, T, H, Hv, d = 1, 4096, 2, 4, 128
    rec = 2 * 4 * (d // 32) * 1024 + 2 * (d // 16) * 1024 + 6 * 1024 + (d // 16) * 4 * 512 + 4 * d
    plain = B * (T // 64) * Hv * rec
    # the workspace holds P = 4 segments' transfer matrices and end states, then
    # one int per record (the exact-decay flags)
    splits = (plain + 255) // 256 * 256 + B * 4 * Hv * d * 2 * d * 4
    assert G().gdr2_chunk_fwd_workspace_bytes(B, T, Hv, d, d, 0, G().GDR2_BF16) == \
        (splits + 255) // 256 * 256 + B * (T // 64) * Hv * 4
    wl = I.make_block(B, T, H, Hv, d, d, s0_std=0.1, seed=45)
    o, ST = run_block(wl, b_scale=2.0)
    ro, rS = oracle_block(wl, b_scale=2.0)
    check(o, ST, ro, rS, "grouped heads, split chains")


@pytest.mark.parametrize("flags", [0, 1, 2, 4, 3, 6])
def test_block_flag_subsets(flags):
    """Each prologue step alone and in pairs; steps that are off take the
    tensors as the operator's inputs (activated gates: sigmoid of the draws;
    log-decay: -softplus of the draws; q, k: already normalised)."""
    wl = I.make_block(2, 150, 2, 4, 64, 64, s0_std=0.1, seed=40 + flags)
    if not flags & 1:
        wl.q = torch.nn.functional.normalize(wl.q.float(), dim=-1).to(torch.bfloat16)
        wl.k = torch.nn.functional.normalize(wl.k.float(), dim=-1).to(torch.bfloat16)
    if not flags & 2:
        wl.f = (-torch.nn.functional.softplus(wl.f.float() - 2.0)).to(wl.f.dtype)
    if not flags & 4:
        wl.b = torch.sigmoid(wl.b.float()).to(torch.bfloat16)
        wl.w = torch.sigmoid(wl.w.float()).to(torch.bfloat16)
    o, ST = run_block(wl, flags=flags)
    ro, rS = oracle_block(wl, flags=flags)
    check(o, ST, ro, rS, f"flags {flags}")


def test_block_without_prologue_is_the_plain_forward():
    """flags = 0 and Hv = H runs the same kernels as gdr2_chunk_fwd: identical bits."""
    wl = I.make_forward(2, 211, 3, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seed=50)
    args = [x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    o1, S1 = G().gdr2_chunk_fwd(*args, wl.S0.cuda())
    o2, S2 = G().gdr2_chunk_fwd_block(*args, flags=0, S0=wl.S0.cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_block_group_members_with_equal_values_agree():
    """Two value heads of one group with the same v and w read the same key
    head, so their outputs and states are identical bit for bit."""
    wl = I.make_block(1, 190, 2, 4, 128, 128, s0_std=0.0, seed=51)
    wl.v[:, :, 3] = wl.v[:, :, 2]
    wl.w[:, :, 3] = wl.w[:, :, 2]
    o, ST = run_block(wl)
    assert torch.equal(o[:, :, 3], o[:, :, 2]) and torch.equal(ST[:, 3], ST[:, 2])
    assert not torch.equal(o[:, :, 1], o[:, :, 2])


def test_block_varlen():
    lens = [1, 0, 70, 64, 129, 3, 200]
    wl = I.make_block(1, sum(lens), 2, 4, 128, 128, s0_std=0.1, seqlens=lens, seed=52)
    o, ST = run_block(wl, b_scale=2.0)
    ro, rS = oracle_block(wl, b_scale=2.0)
    check(o, ST, ro, rS, "block varlen")


@pytest.mark.parametrize("H,Hv", [(16, 16), (8, 16)])
def test_block_full_size(H, Hv):
    """The training shape (B4 T4096, d128) from projections, in the benchmark's
    launch configuration, against the oracle on every (sequence, value head)
    chain."""
    wl = I.make_block(4, 4096, H, Hv, 128, 128, seed=53 + H)
    o, ST = run_block(wl)
    ro, rS = oracle_block(wl)
    check(o, ST, ro, rS, f"block full size H{H} Hv{Hv}, all chains")
