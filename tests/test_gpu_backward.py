"""Backward on the GPU against the fp64 backward oracle (oracle.bwd), through
the C ABI (needs an MI355X).

The backward computes in fp32 from the stored inputs (converted exactly), so
the bar is the fp32 one: max |x - ref| / max |ref| <= 1e-4 per gradient
tensor.  Cases span several chunks with ragged tails, all head sizes the
library supports, packed sequences with zero- and one-token members, and the
training shape on every (sequence, head) chain.
"""
import numpy as np
import pytest
import torch

import gdr2_inputs as I
import oracle
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL = 1e-4
NAMES = {"dq": "dq", "dk": "dk", "dv": "dv", "dlog_alpha": "dg", "db": "db", "dw": "dw"}


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def run_bwd(wl, dO, dST, **kw):
    dev = lambda x: None if x is None else x.cuda()
    out = G().gdr2_chunk_bwd(*(x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                             dO.cuda(), dev(wl.S0), dev(dST), dev(wl.cu_seqlens), **kw)
    torch.cuda.synchronize()
    return {n: None if t is None else t.cpu() for n, t in out.items()}


def oracle_bwd(wl, dO, dST, mask=None):
    cu = None if wl.cu_seqlens is None else wl.cu_seqlens.numpy()
    return oracle.bwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, dO, S0=wl.S0, dST=dST,
                      cu_seqlens=cu, mask=mask)


def check(gr, ref, what, rows=None, with_ds0=True):
    errs = {}
    for ours, theirs in NAMES.items():
        x, r = M.as64(gr[ours]), ref[theirs]
        if rows is not None:
            x, r = rows(x), rows(r)
        errs[ours] = M.max_rel(x, r)
    if with_ds0 and gr["dS0"] is not None:
        errs["dS0"] = M.max_rel(gr["dS0"], ref["dS0"])
    M.record(what, **errs)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, f"{what}: " + ", ".join(f"{n} {e:.3e}" for n, e in bad.items())


@pytest.mark.parametrize("B,T,H,dk,dv,dtype", [
    (2, 150, 2, 64, 64, torch.float32),
    (1, 200, 3, 128, 128, torch.bfloat16),
    (2, 77, 2, 32, 64, torch.bfloat16),
    (1, 64, 2, 128, 32, torch.float32),
    (2, 130, 1, 64, 128, torch.bfloat16),
])
def test_backward_matches_oracle(B, T, H, dk, dv, dtype):
    wl = I.make_forward(B, T, H, dk, dv, dtype=dtype, decay_shift=-2.0, erase_scale=2.0,
                        s0_std=0.1, seed=70 + T + dk)
    dO, dST = I.cotangents(wl, seed=71 + dv)
    check(run_bwd(wl, dO, dST), oracle_bwd(wl, dO, dST), f"B{B} T{T} H{H} dk{dk} dv{dv} {dtype}")


@pytest.mark.parametrize("dtype,la_dtype", [(torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
def test_backward_log_alpha_in_its_own_dtype(dtype, la_dtype):
    """log_alpha in a dtype of its own: fp32 log-decay with bf16 activations, and
    the reverse (the front pass reads each in its own width)."""
    wl = I.make_forward(2, 130, 2, 64, 64, dtype=dtype, la_dtype=la_dtype, decay_shift=-2.0,
                        erase_scale=2.0, s0_std=0.1, seed=76)
    dO, dST = I.cotangents(wl, seed=77)
    check(run_bwd(wl, dO, dST), oracle_bwd(wl, dO, dST), f"{dtype} with log_alpha {la_dtype}")


def test_backward_without_state_arguments():
    """S0 = NULL and dS_T = NULL mean zeros; dS0 may be skipped."""
    wl = I.make_forward(1, 100, 2, 64, 64, dtype=torch.bfloat16, decay_shift=-2.0, seed=72)
    dO, _ = I.cotangents(wl, seed=73)
    gr = run_bwd(wl, dO, None, want_dS0=False)
    check(gr, oracle_bwd(wl, dO, None), "no state arguments", with_ds0=False)
    assert gr["dS0"] is None


def test_backward_packed_sequences():
    lens = [1, 0, 70, 64, 129, 3, 200]
    wl = I.make_forward(1, sum(lens), 2, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=74)
    dO, dST = I.cotangents(wl, seed=75)
    check(run_bwd(wl, dO, dST), oracle_bwd(wl, dO, dST), "packed sequences")


def test_backward_empty_sequence_passes_state_gradient():
    wl = I.make_forward(2, 0, 2, 64, 64, dtype=torch.float32, s0_std=0.1, seed=76)
    dO, dST = I.cotangents(wl, seed=77)
    gr = run_bwd(wl, dO, dST)
    assert torch.equal(gr["dS0"], dST)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_cotangent_scaling_is_exact(dtype):
    """The gradients are linear in (dL/do, dL/dS_T), and every product of the
    backward has one factor that carries the cotangents and one that does not.
    Scaling both cotangents by 2^a therefore scales every gradient by exactly
    2^a, bit for bit, as long as nothing overflows or leaves the normal range:
    the bf16 hi/lo split of an operand commutes with a power-of-two scale, so
    the three-product path has the range of fp32.  Checked at a = 64 and -40
    (gradients near 1e19 and 1e-12 times their unscaled size)."""
    wl = I.make_forward(1, 200, 2, 128, 128, dtype=dtype, s0_std=0.1, seed=79)
    dO, dST = I.cotangents(wl, seed=80)
    base = run_bwd(wl, dO, dST)
    for a in (64, -40):
        f = 2.0 ** a
        gr = run_bwd(wl, (dO.float() * f).to(dO.dtype), dST * f)
        for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0"):
            assert torch.isfinite(gr[n]).all(), (a, n)
            assert torch.equal(gr[n], base[n] * f), (a, n, (gr[n] - base[n] * f).abs().max().item())


def test_backward_training_shape():
    """B4 T4096 H16 d128 bf16 (the benchmark's forward workload) with random
    cotangents, against the oracle on every (sequence, head) chain."""
    wl = I.config(1)
    dO, dST = I.cotangents(wl, seed=78)
    gr = run_bwd(wl, dO, dST)
    check(gr, oracle_bwd(wl, dO, dST), "backward training shape, all chains")
