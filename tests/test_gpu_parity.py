"""GPU path vs the fp64 oracle on the same seeded inputs (needs an MI355X).

Every call goes through the C ABI (the ctypes binding).  Small cases span
several 64-token chunks, ragged tails, packed sequences with zero and one
token, all supported head sizes and both value-block widths; the full-size
workloads run in the launch configuration the benchmark times and are checked
on every (sequence, head) chain.

Tolerances: fp32 path max relative error <= 1e-4 on o and S_T; bf16 path
max-abs error / RMS <= 2e-2 on S_T and on an fp32-stored o, and on a
bf16-stored o beyond its own storage rounding (tests/metrics.py).
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


def dev(x):
    return None if x is None else x.cuda()


def run_fwd(wl, **kw):
    o, ST = G().gdr2_chunk_fwd(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.log_alpha), dev(wl.b),
                               dev(wl.w), dev(wl.S0), dev(wl.cu_seqlens), **kw)
    torch.cuda.synchronize()
    return o.cpu(), None if ST is None else ST.cpu()


def run_fwd_f32_out(wl):
    """The same forward with o stored in fp32 (gdr2_chunk_fwd_f32_out)."""
    return run_fwd(wl, o_dtype=torch.float32)


def oracle_fwd(wl, mask=None):
    cu = None
    if wl.cu_seqlens is not None:
        cu = wl.cu_seqlens.numpy()
    return oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0, cu_seqlens=cu,
                      mask=mask)


def check(o, ST, ro, rS, bf16, what=""):
    """bf16 inputs: S_T and an fp32-stored o are held to the plain max-abs / RMS
    bar; a bf16-stored o to the same bar beyond its own storage rounding, with
    the plain figure recorded beside it.  fp32 inputs: max relative error."""
    if bf16:
        es = M.rms_err(ST, rS)
        plain = M.rms_err(o, ro)
        if o.dtype == torch.bfloat16:
            eo = M.bf16_excess(o, ro)
            M.record(what, o_beyond_bf16_rounding=eo, o_plain=plain,
                     o_bf16_rounding_floor=M.bf16_rounding_floor(ro), S_T=es)
            assert eo <= TOL_BF16 and es <= TOL_BF16, \
                f"{what}: o beyond rounding {eo:.3e} (plain {plain:.3e}), S_T {es:.3e}"
        else:
            eo = plain
            M.record(what, o_plain_f32=plain, S_T=es)
            assert eo <= TOL_BF16 and es <= TOL_BF16, f"{what}: o (fp32) {eo:.3e}, S_T {es:.3e}"
    else:
        eo, es = M.max_rel(o, ro), M.max_rel(ST, rS)
        M.record(what, o_max_rel=eo, S_T_max_rel=es)
        assert eo <= TOL_F32 and es <= TOL_F32, f"{what}: o {eo:.3e}, S_T {es:.3e}"
    return eo, es


# ---- fp32 path: the tiny workload and its collapses --------------------------------

@pytest.mark.parametrize("variant", ["none", "kda", "gdn"])
def test_cfg0_fp32(variant):
    wl = I.config(0, variant=variant)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, False, wl.name)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 32), (32, 128), (64, 64), (128, 128), (128, 32),
                                   (64, 128)])
def test_fp32_shapes_ragged(dk, dv):
    wl = I.make_forward(2, 203, 3, dk, dv, dtype=torch.float32, decay_shift=0.0, s0_std=0.1,
                        seed=11)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, False, f"fp32 dk={dk} dv={dv}")


def test_fp32_d128_b2_t333_h4():
    """fp32 inputs at dk = dv = 128, the pages' head size, with S0 and a fp32
    log-decay: max relative error <= 1e-4 against the oracle."""
    wl = I.make_forward(2, 333, 4, 128, 128, dtype=torch.float32, decay_shift=-2.0, s0_std=0.1,
                        seed=24)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, False, "fp32 B2 T333 H4 d128")


def test_fp32_varlen_and_bf16_log_alpha():
    lens = [1, 63, 0, 65, 130, 7]
    wl = I.make_forward(1, sum(lens), 3, 128, 64, dtype=torch.float32, la_dtype=torch.bfloat16,
                        decay_shift=-2.0, s0_std=0.1, seqlens=lens, seed=25)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, False, "fp32 packed, bf16 log_alpha")
    assert torch.equal(ST[2], wl.S0[2])


# ---- bf16 path --------------------------------------------------------------------

@pytest.mark.parametrize("dk,dv,H", [(128, 128, 4), (128, 128, 64), (64, 128, 4), (32, 64, 8),
                                     (128, 32, 4)])
def test_bf16_shapes_ragged(dk, dv, H):
    # H=4 uses 16-channel value blocks, H=64 the 32-channel ones
    wl = I.make_forward(2, 333, H, dk, dv, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seed=12)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, True, f"bf16 dk={dk} dv={dv} H={H}")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (32, 32)])
def test_bf16_many_chains(dk, dv):
    """256 (sequence, head) chains, one per CU: the state pass runs one
    workgroup per chain over every value channel (two column tiles per
    wavefront); 150 tokens leave a ragged last chunk."""
    wl = I.make_forward(32, 150, 8, dk, dv, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seed=23)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, True, f"256 chains dk={dk} dv={dv}")


def test_bf16_negative_eigenvalues_fp32_decay():
    wl = I.make_forward(1, 700, 4, 128, 128, dtype=torch.bfloat16, la_dtype=torch.float32,
                        decay_shift=-4.0, erase_scale=2.0, s0_std=0.1, seed=13)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, True, "b in [0,2], fp32 log_alpha")


def test_bf16_varlen_edges():
    lens = [1, 63, 64, 65, 0, 130, 7, 200]
    wl = I.make_forward(1, sum(lens), 4, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=14)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, True, "varlen edges")
    # zero-length sequence: S_T = S0 exactly
    assert torch.equal(ST[4], wl.S0[4])


def test_bf16_many_packed_sequences():
    """More sequences than the longest-first sort handles (4096): the state pass
    runs them in index order and the chunk table's prefix sum carries across
    several blocks of 1024 sequences."""
    gen = np.random.default_rng(20)
    lens = [int(x) for x in gen.choice([0, 1, 2, 3, 65], size=4200, p=[0.1, 0.3, 0.3, 0.25, 0.05])]
    wl = I.make_forward(1, sum(lens), 2, 32, 32, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=19)
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, True, "4200 packed sequences")
    zero = [n for n, L in enumerate(lens) if L == 0]
    assert torch.equal(ST[zero], wl.S0[zero])


def test_bf16_without_final_state():
    wl = I.make_forward(2, 150, 3, 64, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seed=22)
    o, ST = run_fwd(wl, want_state=False)
    assert ST is None
    ro, rS = oracle_fwd(wl)
    assert M.bf16_excess(o, ro) <= TOL_BF16


def test_varlen_equals_separate_calls():
    lens = [70, 5, 129]
    wl = I.make_forward(1, sum(lens), 2, 64, 64, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=15)
    o, ST = run_fwd(wl)
    cu = wl.cu_seqlens.tolist()
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        part = I.Workload("part", *(x[:, sl].contiguous() for x in
                                    (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                          wl.S0[n:n + 1].contiguous(), None, 0)
        op, Sp = run_fwd(part)
        assert torch.equal(op, o[:, sl]) and torch.equal(Sp[0], ST[n])


def test_split_resume():
    wl = I.make_forward(1, 256, 4, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seed=16)
    o, ST = run_fwd(wl)
    a = I.Workload("a", *(x[:, :128].contiguous() for x in (wl.q, wl.k, wl.v, wl.log_alpha,
                                                            wl.b, wl.w)), wl.S0, None, 0)
    oa, Sa = run_fwd(a)
    b = I.Workload("b", *(x[:, 128:].contiguous() for x in (wl.q, wl.k, wl.v, wl.log_alpha,
                                                            wl.b, wl.w)), Sa, None, 0)
    ob, Sb = run_fwd(b)
    # chunk boundaries coincide, so the two runs do the same arithmetic
    assert torch.equal(torch.cat([oa, ob], 1), o) and torch.equal(Sb, ST)


def test_deterministic():
    wl = I.make_forward(2, 300, 8, 128, 128, dtype=torch.bfloat16, s0_std=0.1, seed=17)
    o1, S1 = run_fwd(wl)
    o2, S2 = run_fwd(wl)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_state_aliasing_in_place():
    wl = I.make_forward(1, 150, 2, 64, 64, dtype=torch.bfloat16, s0_std=0.1, seed=18)
    o, ST = run_fwd(wl)
    S = dev(wl.S0).clone()
    G().gdr2_chunk_fwd(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.log_alpha), dev(wl.b), dev(wl.w),
                       S, None, S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), ST)


# ---- the full-size workloads, every chain -----------------------------------------

@pytest.mark.parametrize("index", [1, 3, 4])
def test_full_workload(index):
    """Configs 1 (B4 T4096 H16), 3 (B1 T32768 H16, b in [0, 2], S0) and 4 (64
    packed sequences, about 262K tokens), in the launch configuration the
    benchmark times, against the oracle on every (sequence, head) chain: o
    stored in bf16 (beyond its rounding) and in fp32 (plain), and S_T."""
    wl = I.config(index)
    o, ST = run_fwd(wl)
    o32, ST32 = run_fwd_f32_out(wl)
    assert torch.equal(ST32, ST)  # the output's storage type changes nothing else
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, True, f"{wl.name} full, bf16 o")
    check(o32, ST32, ro, rS, True, f"{wl.name} full, fp32 o")
    # a bf16 o is the fp32 o rounded once
    assert torch.equal(o32.to(torch.bfloat16), o)


# ---- strong decay -------------------------------------------------------------------

@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 32),
                                         (torch.float32, 64, 64)])
def test_strong_decay(dtype, dk, dv):
    """Per-token log-decay around -5 (alpha ~ 0.007): 32 consecutive tokens sum
    to about -180, far past the range of one centre per chunk, while any 8
    tokens stay above -80 as the per-block centring needs."""
    wl = I.make_forward(2, 333, 3, dk, dv, dtype=dtype, decay_shift=5.0, s0_std=0.1, seed=60)
    g = wl.log_alpha.double().numpy()
    c = np.concatenate([np.zeros((2, 1) + g.shape[2:]), np.cumsum(g, axis=1)], axis=1)
    assert (c[:, 32:] - c[:, :-32]).min() < -150 and (c[:, 8:] - c[:, :-8]).min() > -80
    o, ST = run_fwd(wl)
    ro, rS = oracle_fwd(wl)
    check(o, ST, ro, rS, dtype == torch.bfloat16, f"strong decay {dtype} dk={dk} dv={dv}")


# ---- decode -------------------------------------------------------------------------

@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.float32), (32, 64, torch.float32),
                                         (64, 32, torch.bfloat16), (128, 128, torch.bfloat16)])
def test_decode_small(dk, dv, dtype):
    N, H = 5, 3
    S = I.decode_state(N, H, dk, dv, seed=21)
    Sd = S.cuda()
    Sr = S.double().numpy()
    for step in range(6):
        x = I.decode_step_inputs(step, N, H, dk, dv, dtype=dtype, seed=21)
        o = G().gdr2_decode_step(*(t.cuda() for t in x), Sd)
        ro, Sr = oracle.decode(*x, Sr)
        torch.cuda.synchronize()
        tol = 1e-4 if dtype == torch.float32 else 1e-2
        assert M.max_rel(o, ro) <= tol, f"step {step} o {M.max_rel(o, ro):.3e}"
        assert M.max_rel(Sd, Sr) <= 1e-4, f"step {step} S {M.max_rel(Sd, Sr):.3e}"


def test_decode_workload_512_steps():
    """Config 2: 256 sequences x 16 heads, 512 in-place steps on the GPU; the oracle
    follows every (sequence, head) chain, and the state and that step's output are
    compared every 64 steps."""
    S = I.decode_state()
    Sd = S.cuda()
    Sr = np.ascontiguousarray(S.double().numpy())
    worst_o = worst_s = 0.0
    for step in range(I.DECODE_STEPS):
        x = I.decode_step_inputs(step)
        o = G().gdr2_decode_step(*(t.cuda() for t in x), Sd)
        ro, _ = oracle.decode(*x, Sr, inplace=True)
        if (step + 1) % 64 == 0:
            torch.cuda.synchronize()
            eo = M.max_rel(o, ro)
            es = M.max_rel(Sd, Sr)
            worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
            assert eo <= TOL_F32 and es <= TOL_F32, f"step {step}: o {eo:.3e} S {es:.3e}"
    M.record("cfg2 decode 512 steps, all chains", o_max_rel=worst_o, S_max_rel=worst_s)


def test_repeated_launches_identical():
    """Regression: the output tile once summed a K=32 and a K=16 MFMA chain in one
    accumulator, which corrupted two of its four registers on some launches.
    Twelve launches into NaN-filled outputs must all equal the first, bit for bit,
    and the first must meet the tolerance."""
    wl = I.make_forward(2, 333, 64, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seed=12)
    args = [dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, wl.S0)]
    first = None
    for rep in range(12):
        o = torch.full((2, 333, 64, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        _, ST = G().gdr2_chunk_fwd(*args, o=o)
        torch.cuda.synchronize()
        if first is None:
            first = (o.cpu(), ST.cpu())
            ro, rS = oracle_fwd(wl)
            check(first[0], first[1], ro, rS, True, "repeat launch 0")
        else:
            assert torch.equal(o.cpu(), first[0]) and torch.equal(ST.cpu(), first[1]), f"launch {rep}"
