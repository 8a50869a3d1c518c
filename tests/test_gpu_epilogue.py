"""Output epilogue on the GPU (RMSNorm, then a SiLU output gate) against the
fp64 oracle, through the C ABI (needs an MI355X).

Tolerance, from the arithmetic: the kernel works in fp32.  The sum of squares
over a group of n channels carries at most n rounding errors (relative n*u,
u = 2^-24), which the reciprocal square root halves; the square root itself,
exp, the reciprocal in the sigmoid and the four products add at most about 16
more.  So the fp32 value is within (n/2 + 16) u of the exact result, relative
per element; the bf16 output then adds its own storage rounding (half a bf16
ulp).  An absolute floor of 1e-37 covers gate values whose sigmoid underflows
in fp32 (z = -100 gives 0 instead of about 4e-42).
"""
import numpy as np
import pytest
import torch

import gdr2_inputs as I
import oracle
from oracle import epilogue as E
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

U = 2.0 ** -24


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def check_elementwise(y, ref, group, bf16, what=""):
    y, ref = M.as64(y), M.as64(ref)
    rel = (group / 2 + 16) * U
    tol = rel * np.abs(ref) + 1e-37
    if bf16:
        tol = tol + M.bf16_half_ulp(np.maximum(np.abs(ref), np.abs(y)))
    err = np.abs(y - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of bound, worst at "
                           f"{np.unravel_index(np.argmax(err - tol), err.shape)}: "
                           f"y={y[bad][0]!r} ref={ref[bad][0]!r}")


def run(o, z, wt, eps, group, **kw):
    y = G().gdr2_norm_gate(o.cuda(), z.cuda(), None if wt is None else wt.cuda(), eps, group, **kw)
    torch.cuda.synchronize()
    return y


# (shape, group): per-head over dv, whole row, per-head groups inside a row with
# a per-head weight, small and odd groups (idle lanes), and groups of 2 to 16
# chunks per lane
CASES = [
    ((2, 77, 4, 128), 128), ((2, 77, 4, 64), 64), ((3, 50, 2, 32), 32),
    ((2, 77, 4 * 128), 4 * 128), ((2, 77, 4 * 128), 128),
    ((1000, 8), 8), ((333, 24), 24), ((101, 3 * 40), 40), ((37, 96), 96),
    ((19, 1024), 1024), ((9, 2048), 2048), ((5, 4096), 4096), ((3, 8192), 8192),
    ((4, 8192), 2048),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("shape,group", CASES, ids=lambda x: str(x))
def test_norm_gate_matches_oracle(shape, group, dtype):
    o, z, wt = I.epilogue_inputs(shape, dtype=dtype, seed=len(shape) * 1000 + group)
    y = run(o, z, wt, 1e-6, group)
    ref = E.norm_gate(o, z, wt, eps=1e-6, group=group)
    check_elementwise(y.cpu(), ref, group, dtype == torch.bfloat16, f"{shape} group {group}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_norm_gate_edges(dtype):
    """No weight, eps = 0, zero rows with eps > 0, and gates at +-100."""
    o, z, _ = I.epilogue_inputs((64, 128), dtype=dtype, seed=7, weight=False)
    check_elementwise(run(o, z, None, 0.0, 128).cpu(), E.norm_gate(o, z, None, eps=0.0), 128,
                      dtype == torch.bfloat16, "no weight, eps 0")
    o[5] = 0
    z[9, :4] = 100.0
    z[9, 4:8] = -100.0
    y = run(o, z, None, 1e-5, 128).cpu()
    assert torch.all(y[5] == 0)
    check_elementwise(y, E.norm_gate(o, z, None, eps=1e-5), 128, dtype == torch.bfloat16,
                      "zero row, saturated gate")


def test_norm_gate_in_place():
    o, z, wt = I.epilogue_inputs((4, 333, 16, 128), seed=9)
    ref = E.norm_gate(o, z, wt, eps=1e-6, group=128)
    od, zd, wd = o.cuda(), z.cuda(), wt.cuda()
    G().gdr2_norm_gate(od, zd, wd, 1e-6, 128, y=od)     # over o
    torch.cuda.synchronize()
    check_elementwise(od.cpu(), ref, 128, True, "y = o")
    od = o.cuda()
    G().gdr2_norm_gate(od, zd, wd, 1e-6, 128, y=zd)     # over z
    torch.cuda.synchronize()
    check_elementwise(zd.cpu(), ref, 128, True, "y = z")


def test_norm_gate_empty():
    o = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    y = G().gdr2_norm_gate(o, o.clone(), None, 1e-6)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


def test_norm_gate_after_forward_full_size():
    """The epilogue on the forward's own output at the training shape (B4 T4096
    H16 d128, bf16), per head over dv, in place on o: every row is checked
    against the oracle applied to the stored o."""
    wl = I.config(1)
    o, _ = G().gdr2_chunk_fwd(*(x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                              want_state=False)
    torch.cuda.synchronize()
    o_stored = o.cpu()
    _, z, wt = I.epilogue_inputs(tuple(o.shape), seed=11)
    G().gdr2_norm_gate(o, z.cuda(), wt.cuda(), 1e-6, 128, y=o)
    torch.cuda.synchronize()
    ref = E.norm_gate(o_stored, z, wt, eps=1e-6, group=128)
    check_elementwise(o.cpu(), ref, 128, True, "forward + epilogue")


# ---- decode with the epilogue fused into its store -----------------------------------

@pytest.mark.parametrize("dk,dv,dtype,weight", [
    (128, 128, torch.float32, True), (32, 64, torch.float32, False),
    (64, 32, torch.bfloat16, True), (128, 128, torch.bfloat16, True),
    (128, 64, torch.bfloat16, False)])
def test_decode_norm_gate_small(dk, dv, dtype, weight):
    """Several steps: the state must match the plain decode step bit for bit and
    y must match the oracle's decode followed by the oracle's epilogue."""
    N, H = 5, 3
    S = I.decode_state(N, H, dk, dv, seed=23)
    Sg, Sp = S.cuda(), S.cuda()
    Sr = S.double().numpy()
    wt = (1 + 0.1 * torch.randn(dv, generator=torch.Generator().manual_seed(3))) if weight else None
    for step in range(5):
        x = I.decode_step_inputs(step, N, H, dk, dv, dtype=dtype, seed=23)
        _, z, _ = I.epilogue_inputs((N, H, dv), dtype=dtype, seed=500 + step, weight=False)
        y = G().gdr2_decode_step_norm_gate(*(t.cuda() for t in x), Sg, z.cuda(),
                                           None if wt is None else wt.cuda(), 1e-6)
        G().gdr2_decode_step(*(t.cuda() for t in x), Sp)
        ro, Sr = oracle.decode(*x, Sr)
        ry = E.norm_gate(ro, z, wt, eps=1e-6)
        torch.cuda.synchronize()
        assert torch.equal(Sg, Sp), f"step {step}: state differs from the plain decode step"
        # o itself carries the decode step's fp32 error (max_rel <= 1e-4 of the
        # output's scale); the epilogue rescales each head to unit RMS
        err = M.rms_err(y, ry) if dtype == torch.float32 else M.bf16_excess(y, ry)
        tol = 1e-4 if dtype == torch.float32 else 1e-2
        assert err <= tol, f"step {step}: y error {err:.3e}"


def test_decode_norm_gate_workload_sampled():
    """The decode workload (256 sequences x 16 heads, d128, fp32) for 64 fused
    steps with y written over z; the oracle follows 8 sequences."""
    S = I.decode_state()
    Sd = S.cuda()
    seqs = [0, 37, 101, 128, 199, 200, 254, 255]
    Sr = S[seqs].double().numpy()
    wt = 1 + 0.1 * torch.randn(128, generator=torch.Generator().manual_seed(4))
    wd = wt.cuda()
    for step in range(64):
        x = I.decode_step_inputs(step)
        _, z, _ = I.epilogue_inputs((256, 16, 128), dtype=torch.float32, seed=700 + step,
                                    weight=False)
        zd = z.cuda()
        G().gdr2_decode_step_norm_gate(*(t.cuda() for t in x), Sd, zd, wd, 1e-6, y=zd)
        ro, Sr = oracle.decode(*(t[seqs] for t in x), Sr)
        if (step + 1) % 16 == 0:
            torch.cuda.synchronize()
            ry = E.norm_gate(ro, z[seqs], wt, eps=1e-6)
            ey, es = M.rms_err(zd[seqs], ry), M.max_rel(Sd[seqs], Sr)
            assert ey <= 1e-4 and es <= 1e-4, f"step {step}: y {ey:.3e} S {es:.3e}"
