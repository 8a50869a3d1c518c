"""Strong decay on the GPU path: per-token log-decay down to -100 (alpha ~ 4e-44),
where the decay factors of the chunk matrices leave every floating-point range
(needs an MI355X).

The log-decay of the operator is any g <= 0 (Gated DeltaNet-2 pages, "Gate
Parameterization", Eq. 12: -exp(a) softplus(.) is unbounded below, and alpha
-> 0 forgets everything).  Chunks whose decay centred factors cannot carry
take the exact path of each kernel (entry by entry, with the exact decay);
the others keep the factored products.  The cases mix both inside one call.
Bars: the path's own (fp32: max relative error 1e-4; bf16: max-abs error over
the RMS 2e-2, o beyond its bf16 rounding), against the fp64 oracle; an fp32
gradient whose exact values all lie below the fp32 range (they carry the
decay e^-100 itself) is held to an absolute error of 2^-126 (tests/metrics.py).
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

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
NAMES = {"dq": "dq", "dk": "dk", "dv": "dv", "dlog_alpha": "dg", "db": "db", "dw": "dw"}


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def dev(x):
    return None if x is None else x.cuda()


def with_decay(wl, g, frac=1.0, seed=0):
    """Set log_alpha to the constant g on a random fraction of the (token, head,
    channel) entries (all of them when frac = 1), keeping the rest."""
    la = wl.log_alpha.float()
    if frac >= 1.0:
        la = torch.full_like(la, g)
    else:
        gen = torch.Generator("cpu").manual_seed(seed)
        pick = torch.rand(la.shape, generator=gen) < frac
        la = torch.where(pick, torch.full_like(la, g), la)
    wl.log_alpha = la.to(wl.log_alpha.dtype).contiguous()
    return wl


def check_fwd(wl, what):
    o, ST = G().gdr2_chunk_fwd(*(dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                               dev(wl.S0), dev(wl.cu_seqlens))
    torch.cuda.synchronize()
    o, ST = o.cpu(), ST.cpu()
    cu = None if wl.cu_seqlens is None else wl.cu_seqlens.numpy()
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0, cu_seqlens=cu)
    assert torch.isfinite(o.float()).all() and torch.isfinite(ST).all(), f"{what}: non-finite output"
    if wl.q.dtype == torch.float32:
        eo, es = M.max_rel(o, ro), M.max_rel(ST, rS)
        tol = TOL_F32
    else:
        eo, es = M.bf16_excess(o, ro), M.rms_err(ST, rS)
        tol = TOL_BF16
    M.record(what, o=eo, S_T=es)
    assert eo <= tol and es <= tol, f"{what}: o {eo:.3e}, S_T {es:.3e}"


FWD_CASES = [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 32), (torch.bfloat16, 32, 64),
             (torch.float32, 128, 128), (torch.float32, 64, 64)]


@pytest.mark.parametrize("g", [-20.0, -100.0])
@pytest.mark.parametrize("dtype,dk,dv", FWD_CASES)
def test_forward_constant_strong_decay(g, dtype, dk, dv):
    wl = I.make_forward(2, 203, 3, dk, dv, dtype=dtype, la_dtype=torch.float32, decay_shift=-2.0,
                        s0_std=0.1, seed=110)
    check_fwd(with_decay(wl, g), f"fwd g={g} {dtype} dk{dk} dv{dv}")


@pytest.mark.parametrize("dtype,dk,dv", FWD_CASES)
def test_forward_scattered_strong_decay(dtype, dk, dv):
    """About 1% of the decay entries at -60: some chunks take the exact path and
    some do not, inside one call (packed sequences too)."""
    lens = [70, 0, 129, 5, 200, 64]
    wl = I.make_forward(1, sum(lens), 4, dk, dv, dtype=dtype, la_dtype=torch.float32,
                        decay_shift=-2.0, s0_std=0.1, seqlens=lens, seed=111)
    check_fwd(with_decay(wl, -60.0, frac=0.01, seed=112), f"fwd scattered {dtype} dk{dk} dv{dv}")


def test_forward_strong_decay_full_shape_bf16_log_alpha():
    """The training shape (B4 T4096 H16 d128) with bf16 log-decay at -20 on 2% of
    the entries."""
    wl = I.config(1)
    check_fwd(with_decay(wl, -20.0, frac=0.02, seed=113), "fwd B4 T4096 H16 scattered -20")


@pytest.mark.parametrize("a_scale", [5.0, 8.0])
def test_block_prologue_strong_decay(a_scale):
    """Eq. 12 with large exp(a): -exp(a) softplus(f + delta) reaches -100 and beyond
    per token; grouped value heads."""
    wl = I.make_block(2, 203, 2, 4, 128, 128, s0_std=0.1, seed=114)
    wl.a = wl.a + a_scale
    o, ST = G().gdr2_chunk_fwd_block(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.f), dev(wl.b), dev(wl.w),
                                     dev(wl.a), dev(wl.delta), S0=dev(wl.S0))
    torch.cuda.synchronize()
    o, ST = o.cpu(), ST.cpu()
    ins = P.block_inputs(wl.q, wl.k, wl.v, wl.f, wl.b, wl.w, wl.a, wl.delta)
    assert ins[3].min() < -100
    ro, rS = oracle.fwd(*ins, S0=wl.S0)
    eo, es = M.bf16_excess(o, ro), M.rms_err(ST, rS)
    M.record(f"block strong decay a+{a_scale}", o=eo, S_T=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16, f"o {eo:.3e}, S_T {es:.3e}"


def check_bwd(wl, what, seed=115):
    dO, dST = I.cotangents(wl, seed=seed)
    out = G().gdr2_chunk_bwd(*(x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                             dO.cuda(), dev(wl.S0), dev(dST), dev(wl.cu_seqlens))
    torch.cuda.synchronize()
    cu = None if wl.cu_seqlens is None else wl.cu_seqlens.numpy()
    ref = oracle.bwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, dO, S0=wl.S0, dST=dST,
                     cu_seqlens=cu)
    # gradients that carry the decay itself (db, dlog_alpha, dS0 under alpha ~
    # e^-100) lie below the fp32 range: their bar bottoms out at FP32_TINY
    floor = M.FP32_TINY / TOL_F32
    errs = {n: M.max_rel(out[n].cpu(), ref[r], floor) for n, r in NAMES.items()}
    errs["dS0"] = M.max_rel(out["dS0"].cpu(), ref["dS0"], floor)
    M.record(what, **errs)
    bad = {n: e for n, e in errs.items() if not e <= TOL_F32}
    assert not bad, f"{what}: " + ", ".join(f"{n} {e:.3e}" for n, e in bad.items())


@pytest.mark.parametrize("g", [-20.0, -100.0])
@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 32)])
def test_backward_constant_strong_decay(g, dtype, dk, dv):
    wl = I.make_forward(2, 150, 2, dk, dv, dtype=dtype, la_dtype=torch.float32, decay_shift=-2.0,
                        erase_scale=2.0, s0_std=0.1, seed=116)
    check_bwd(with_decay(wl, g), f"bwd g={g} {dtype} dk{dk} dv{dv}")


def test_backward_scattered_strong_decay():
    lens = [70, 0, 129, 5, 200]
    wl = I.make_forward(1, sum(lens), 3, 128, 64, dtype=torch.bfloat16, la_dtype=torch.float32,
                        decay_shift=-2.0, s0_std=0.1, seqlens=lens, seed=117)
    check_bwd(with_decay(wl, -60.0, frac=0.01, seed=118), "bwd scattered -60")


def test_backward_on_block_gates():
    """The backward on the operator inputs that the block's own prologue makes
    (Eq. 12 decay from make_block's draws, with exp(a) scaled by e so that
    32-token windows reach far below -80), in fp32."""
    bl = I.make_block(2, 256, 2, 2, 128, 128, s0_std=0.1, seed=7)
    bl.a = bl.a + 1.0
    q, k, v, g, b, w = (torch.from_numpy(x).float().contiguous() for x in
                        P.block_inputs(bl.q, bl.k, bl.v, bl.f, bl.b, bl.w, bl.a, bl.delta))
    c = np.concatenate([np.zeros((2, 1, 2, 128)), np.cumsum(g.double().numpy(), axis=1)], axis=1)
    worst32 = (c[:, 32:] - c[:, :-32]).min()
    assert worst32 < -80
    wl = I.Workload("block gates", q, k, v, g, b, w, bl.S0, None, 7)
    check_bwd(wl, f"bwd on block gates (worst 32-token window {worst32:.1f})")
