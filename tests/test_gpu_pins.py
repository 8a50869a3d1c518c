"""Special cases whose results the recurrence fixes in closed form, run on the GPU
path through the C ABI (needs an MI355X).

Each case pins the kernels to something other than the oracle as well as to
it (Gated DeltaNet-2 pages, "The Gated Delta Rule-2 State Update", Eq. 10 and
its Steps 1-5; "Gate Parameterization" for the gate ranges):

* pure decay, b = w = 0: both gate terms of Eq. 10 vanish, so S_t =
  Diag(exp(G_t)) S0 with G_t the cumulative log-decay, and o_t = S_t^T q_t;
* no decay, log_alpha = 0: the chunk matrices carry no decay factors at all;
* the reflector endpoint of the negative-eigenvalue range, b = 2, w = 0,
  alpha = 1 and a unit key: each transition is I - 2 k k^T, orthogonal, so the
  state's Frobenius norm never changes, and a key applied twice in a row
  undoes itself, so a sequence of repeated pairs returns S0;
* the tied-gate collapses (b = w = beta: KDA; additionally a scalar decay:
  Gated DeltaNet) on the bf16 path.

Keys of the reflector case have entries +-1/8 on 64 of 128 channels (+-1/4 on
16 of 32), so their norm is exactly 1 in bf16 as well as in fp32.
Tolerances: the path's own bars (fp32: max relative error 1e-4; bf16: max-abs
error over the reference RMS 2e-2, o beyond its bf16 rounding).
"""
import numpy as np
import pytest
import torch

import gdr2_inputs as I
import oracle
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def run(wl):
    dev = lambda x: None if x is None else x.cuda()
    o, ST = G().gdr2_chunk_fwd(*(dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                               dev(wl.S0), dev(wl.cu_seqlens))
    torch.cuda.synchronize()
    return o.cpu(), ST.cpu()


def bar(x, ref, dtype, what):
    """The path's parity bar between a GPU tensor and a fp64 reference."""
    if dtype == torch.float32:
        e = M.max_rel(x, ref)
        tol = TOL_F32
    elif x.dtype == torch.bfloat16:
        e = M.bf16_excess(x, ref)
        tol = TOL_BF16
    else:
        e = M.rms_err(x, ref)
        tol = TOL_BF16
    M.record(what, err=e)
    assert e <= tol, f"{what}: {e:.3e}"


CASES = [(torch.float32, 64, 64), (torch.float32, 32, 32), (torch.bfloat16, 128, 128),
         (torch.bfloat16, 64, 128), (torch.bfloat16, 32, 64)]


@pytest.mark.parametrize("dtype,dk,dv", CASES)
def test_pure_decay(dtype, dk, dv):
    wl = I.make_forward(2, 203, 3, dk, dv, dtype=dtype, decay_shift=-2.0, s0_std=0.1, seed=90)
    wl.b.zero_()
    wl.w.zero_()
    o, ST = run(wl)
    # closed form: S_t = Diag(exp(G_t)) S0, o_t = S0^T (exp(G_t) * q_t)
    g = wl.log_alpha.double().numpy()
    q = wl.q.double().numpy()
    S0 = wl.S0.double().numpy()
    gam = np.exp(np.cumsum(g, axis=1))                        # [B, T, H, dk]
    o_ref = np.einsum("bthi,bhij->bthj", gam * q, S0)
    S_ref = gam[:, -1][..., None] * S0
    bar(o, o_ref, dtype, f"pure decay o {dtype} dk{dk} dv{dv}")
    bar(ST, S_ref, dtype if dtype == torch.float32 else None, f"pure decay S_T {dtype} dk{dk} dv{dv}")
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    assert np.abs(ro - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
    assert np.abs(rS - S_ref).max() <= 1e-12 * max(1.0, np.abs(S_ref).max())


@pytest.mark.parametrize("dtype,dk,dv", CASES)
def test_no_decay(dtype, dk, dv):
    wl = I.make_forward(2, 203, 3, dk, dv, dtype=dtype, decay_shift=-2.0, s0_std=0.1, seed=91)
    wl.log_alpha.zero_()
    o, ST = run(wl)
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    bar(o, ro, dtype, f"no decay o {dtype} dk{dk} dv{dv}")
    bar(ST, rS, dtype if dtype == torch.float32 else None, f"no decay S_T {dtype} dk{dk} dv{dv}")


def unit_keys(gen, B, T, H, dk, dtype):
    """Unit keys exact in bf16: +-1/8 on 64 random channels of 128, or +-1/4 on
    16 random channels (dk = 32 or 64), so the squares sum to exactly 1."""
    nz, val = {128: (64, 0.125), 64: (16, 0.25), 32: (16, 0.25)}[dk]
    k = torch.zeros(B, T, H, dk)
    for idx in np.ndindex(B, T, H):
        ch = torch.randperm(dk, generator=gen)[:nz]
        sg = torch.randint(0, 2, (nz,), generator=gen).float() * 2 - 1
        k[idx][ch] = sg * val
    return k.to(dtype)


@pytest.mark.parametrize("dtype,dk,dv", CASES)
def test_reflector_endpoint(dtype, dk, dv):
    B, T, H = 2, 202, 2
    wl = I.make_forward(B, T, H, dk, dv, dtype=dtype, decay_shift=0.0, s0_std=0.1, seed=92)
    gen = torch.Generator("cpu").manual_seed(93)
    k = unit_keys(gen, B, T // 2, H, dk, dtype)
    wl.k = k.repeat_interleave(2, dim=1).contiguous()   # every key twice in a row
    wl.b.fill_(2.0)
    wl.w.zero_()
    wl.log_alpha.zero_()
    assert torch.equal((wl.k.double() ** 2).sum(-1), torch.ones(B, T, H, dtype=torch.float64))
    o, ST = run(wl)
    S0 = wl.S0.double().numpy()
    # pairs of equal reflections cancel: S_T = S0
    bar(ST, S0, dtype if dtype == torch.float32 else None, f"reflector S_T = S0 {dtype} dk{dk} dv{dv}")
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    bar(o, ro, dtype, f"reflector o {dtype} dk{dk} dv{dv}")
    # a single reflection keeps the norm: the state after an odd number of tokens
    one = I.Workload("odd", *(x[:, :T - 1].contiguous() for x in
                              (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)), wl.S0, None, 0)
    _, S_odd = run(one)
    n_odd = np.sqrt((S_odd.double().numpy() ** 2).sum(axis=(2, 3)))
    n0 = np.sqrt((S0 ** 2).sum(axis=(2, 3)))
    rel = np.abs(n_odd - n0).max() / n0.max()
    M.record(f"reflector norm {dtype} dk{dk} dv{dv}", err=rel)
    assert rel <= (TOL_F32 if dtype == torch.float32 else TOL_BF16), f"norm drift {rel:.3e}"


@pytest.mark.parametrize("tie", ["kda", "gdn"])
def test_tied_gate_collapses_bf16(tie):
    wl = I.make_forward(2, 203, 4, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        tie=tie, seed=94)
    o, ST = run(wl)
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    bar(o, ro, torch.bfloat16, f"{tie} collapse o bf16")
    bar(ST, rS, None, f"{tie} collapse S_T bf16")
