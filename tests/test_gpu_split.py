"""Split chains of the bf16 forward vs the fp64 oracle (needs an MI355X).

With few long (sequence, head) chains and dk == dv, the forward cuts every
sequence's chunks into P segments: a transfer pass forms each segment's
affine map of its entry state (Eq. 23 of the pages' chunkwise form, composed
over the segment), an fp32 scan chains the maps, and the state pass runs all
segments at once.  Without cu_seqlens the segment plan depends on the shape
only; `plan` below restates it so each case states the P it exercises, and
the workspace size the library asks for confirms that plan.  Packed
sequences (Appendix C.6) are planned on the device from cu_seqlens, each
sequence on its own: `packed_plan` restates that plan, so each packed case
states which sequences it splits.  Tolerance as for the rest of the bf16
path: max-abs error / RMS <= 2e-2 on S_T and on o beyond o's own bf16
storage rounding, and the plain metric on o stored in fp32.
"""
import math

import pytest
import torch

import gdr2_inputs as I
import oracle
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_BF16 = 2e-2


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def dev(x):
    return None if x is None else x.cuda()


def plan(chains, T, dk, dv):
    """Segments per sequence and chunks per segment, as the library plans them."""
    nc = (T + 63) // 64
    if dk != dv or chains >= 64:
        return 1, nc
    P = 1
    while P < 16 and chains * P * 2 <= 256 and nc // (P * 2) >= 16:
        P *= 2
    if P == 1:
        return 1, nc
    segc = -(-nc // P)
    return -(-nc // segc), segc


def rec_bytes(dk, dv):
    return 2 * 4 * (dk // 32) * 1024 + 2 * (dk // 16) * 1024 + 6 * 1024 + (dv // 16) * 4 * 512 + 4 * dk


def assert_split(B, T, H, dk, P):
    """The workspace the library asks for has the transfer matrices and end
    states of P segments per chain exactly when P > 1 (then one int per record
    for the exact-decay flags)."""
    nc = (T + 63) // 64
    rec = B * nc * H * rec_bytes(dk, dk)
    extra = 0 if P == 1 else B * P * H * dk * 2 * dk * 4
    base = (rec + 255) // 256 * 256 if P > 1 else rec
    total = (base + extra + 255) // 256 * 256 + B * nc * H * 4
    assert G().gdr2_chunk_fwd_workspace_bytes(B, T, H, dk, dk, 0, G().GDR2_BF16) == total


def run(wl, **kw):
    o, ST = G().gdr2_chunk_fwd(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.log_alpha), dev(wl.b),
                               dev(wl.w), dev(wl.S0), None, **kw)
    torch.cuda.synchronize()
    return o.cpu(), None if ST is None else ST.cpu()


def check(o, ST, wl, what):
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    eo = M.bf16_excess(o, ro)
    assert eo <= TOL_BF16, f"{what}: o excess {eo:.3e}"
    if ST is not None:
        es = M.rms_err(ST, rS)
        assert es <= TOL_BF16, f"{what}: S_T {es:.3e}"


@pytest.mark.parametrize("B,T,H,dk,P", [
    (1, 4096, 2, 128, 4),            # 64 chunks, 16 per segment
    (1, 64 * 37 + 13, 1, 64, 2),     # 38 chunks: segments of 19, ragged last chunk
    (1, 64 * 130 + 5, 1, 128, 8),    # 131 chunks: 7 segments of 17 and one of 12
    (1, 8192, 1, 32, 8),             # dk = dv = 32, 128 chunks
    (2, 64 * 80, 3, 64, 4),          # 6 chains of 80 chunks, segments of 20
    (1, 16384, 1, 128, 16),          # the largest split: 16 segments of 16 chunks
])
def test_split_chains(B, T, H, dk, P):
    assert plan(B * H, T, dk, dk)[0] == P
    assert_split(B, T, H, dk, P)
    wl = I.make_forward(B, T, H, dk, dk, dtype=torch.bfloat16, decay_shift=-4.0,
                        erase_scale=2.0, s0_std=0.1, seed=70 + P)
    o, ST = run(wl)
    check(o, ST, wl, f"B{B} T{T} H{H} d{dk} P={P}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(ST).all()


def test_split_zero_state_and_no_final_state():
    wl = I.make_forward(1, 4096, 2, 64, 64, dtype=torch.bfloat16, decay_shift=-2.0, seed=80)
    assert wl.S0 is None and plan(2, 4096, 64, 64)[0] == 4
    o, ST = run(wl)
    check(o, ST, wl, "S0 = 0")
    o2, ST2 = run(wl, want_state=False)
    assert ST2 is None and torch.equal(o2, o)


def test_split_state_aliasing_in_place():
    """S_T may alias S0: the last segment writes S_T in the same launch in
    which segment 0 starts, from the copy of S0 the transfer pass keeps."""
    wl = I.make_forward(1, 4096, 2, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seed=81)
    o, ST = run(wl)
    S = dev(wl.S0).clone()
    o2, _ = G().gdr2_chunk_fwd(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.log_alpha), dev(wl.b),
                               dev(wl.w), S, None, S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), ST) and torch.equal(o2.cpu(), o)


def test_split_deterministic_and_close_to_unsplit():
    """Two split runs are bitwise equal, and the same sequence passed as one
    packed sequence (which the device plan cuts into 2 segments of 32 chunks,
    not 4 of 16) agrees to the bf16 tolerance."""
    wl = I.make_forward(1, 4096, 2, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seed=82)
    o1, S1 = run(wl)
    o2, S2 = run(wl)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    cu = torch.tensor([0, 4096], dtype=torch.int32)
    o3, S3 = G().gdr2_chunk_fwd(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.log_alpha), dev(wl.b),
                                dev(wl.w), dev(wl.S0), dev(cu))
    torch.cuda.synchronize()
    assert M.rms_err(S1, S3.cpu()) <= TOL_BF16
    assert M.rms_err(o1.float(), o3.cpu().float()) <= TOL_BF16


# ---- packed sequences -------------------------------------------------------------

PSEG_MIN = 32


def packed_plan(lens, H, slots=256):
    """Segments per sequence of the device's plan for packed sequences (dk ==
    dv, more than 32 chunks in all): ceil(nc / L) with L the largest of 32
    chunks, the chunks x heads per CU and sqrt(2 x the longest sequence's
    chunks)."""
    ncs = [(n + 63) // 64 for n in lens]
    total = sum(ncs)
    L = max(PSEG_MIN, -(-total * H // slots), math.ceil(math.sqrt(2.0 * max(ncs))))
    return [-(-c // L) if c > L else 1 for c in ncs]


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def run_packed(wl, o_f32=False, **kw):
    args = [dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, wl.S0, wl.cu_seqlens)]
    if o_f32:
        o, ST = G().gdr2_chunk_fwd(*args, o_dtype=torch.float32, **kw)
    else:
        o, ST = G().gdr2_chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    return o.cpu(), ST.cpu()


def check_packed(wl, what, f32_too=False):
    o, ST = run_packed(wl)
    cu = wl.cu_seqlens.numpy()
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0, cu_seqlens=cu)
    assert torch.isfinite(o.float()).all() and torch.isfinite(ST).all(), what
    eo, es = M.bf16_excess(o, ro), M.rms_err(ST, rS)
    figs = dict(o_beyond_bf16_rounding=eo, o_plain=M.rms_err(o, ro), S_T=es)
    if f32_too:
        of, _ = run_packed(wl, o_f32=True)
        figs["o_plain_f32"] = M.rms_err(of, ro)
        assert figs["o_plain_f32"] <= TOL_BF16, f"{what}: o (fp32 store) {figs['o_plain_f32']:.3e}"
    M.record(what, **figs)
    assert eo <= TOL_BF16 and es <= TOL_BF16, f"{what}: o excess {eo:.3e}, S_T {es:.3e}"
    return o, ST


def test_packed_long_sequence_among_short_ones():
    """One 32K-token sequence among 63 short ones (U[1, 512] tokens), H16
    d128: the long sequence is cut into segments, the others run whole."""
    gen = torch.Generator("cpu").manual_seed(130)
    lens = [32768] + torch.randint(1, 513, (63,), generator=gen).tolist()
    P = packed_plan(lens, 16, cus())
    assert P[0] > 1 and max(P[1:]) == 1
    wl = I.make_forward(1, sum(lens), 16, 128, 128, dtype=torch.bfloat16, decay_shift=-4.0,
                        erase_scale=2.0, s0_std=0.1, seqlens=lens, seed=131)
    check_packed(wl, f"packed: 32K among 63 short, {P[0]} segments", f32_too=True)


@pytest.mark.parametrize("lens,H,dk", [
    ([0, 9000, 3, 0, 20000, 64, 12000, 1], 2, 64),   # several long ones, empty ones
    ([5000, 40, 7000], 1, 32),                       # dk = dv = 32
    ([4095, 4097, 130 * 64 + 17], 4, 128),          # ragged ends, every sequence split
])
def test_packed_split_cases(lens, H, dk):
    P = packed_plan(lens, H, cus())
    assert max(P) > 1
    wl = I.make_forward(1, sum(lens), H, dk, dk, dtype=torch.bfloat16, decay_shift=-4.0,
                        erase_scale=2.0, s0_std=0.1, seqlens=lens, seed=132 + H)
    check_packed(wl, f"packed split {lens} H{H} d{dk}, segments {P}")


def test_packed_split_without_states_and_aliased():
    """S0 = NULL, S_T not wanted, and S_T aliasing S0 with split sequences: the
    last segment writes S_T in the launch in which segment 0 reads S0."""
    lens = [9000, 17, 6000]
    assert max(packed_plan(lens, 2, cus())) > 1
    wl = I.make_forward(1, sum(lens), 2, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=140)
    o, ST = check_packed(wl, "packed split with S0")
    S = dev(wl.S0).clone()
    args = [dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    o2, _ = G().gdr2_chunk_fwd(*args, S, dev(wl.cu_seqlens), S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(S.cpu(), ST) and torch.equal(o2.cpu(), o)
    wl.S0 = None
    o3, _ = G().gdr2_chunk_fwd(*args, None, dev(wl.cu_seqlens), want_state=False)
    torch.cuda.synchronize()
    ro, _ = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, cu_seqlens=wl.cu_seqlens.numpy())
    assert M.bf16_excess(o3.cpu(), ro) <= TOL_BF16


def test_packed_split_block_grouped_heads():
    """The block forward from projections with packed sequences, grouped value
    heads (Hv = 2H) and a sequence long enough to split."""
    from oracle import prologue as PR
    lens = [6000, 100, 2500]
    wl = I.make_block(1, sum(lens), 2, 4, 128, 128, s0_std=0.1, seqlens=lens, seed=141)
    assert max(packed_plan(lens, 4, cus())) > 1
    o, ST = G().gdr2_chunk_fwd_block(dev(wl.q), dev(wl.k), dev(wl.v), dev(wl.f), dev(wl.b), dev(wl.w),
                                     dev(wl.a), dev(wl.delta), S0=dev(wl.S0), cu_seqlens=dev(wl.cu_seqlens))
    torch.cuda.synchronize()
    ins = PR.block_inputs(wl.q, wl.k, wl.v, wl.f, wl.b, wl.w, wl.a, wl.delta)
    ro, rS = oracle.fwd(*ins, S0=wl.S0, cu_seqlens=wl.cu_seqlens.numpy())
    eo, es = M.bf16_excess(o.cpu(), ro), M.rms_err(ST.cpu(), rS)
    M.record("packed split block Hv=2H", o_beyond_bf16_rounding=eo, S_T=es)
    assert eo <= TOL_BF16 and es <= TOL_BF16, f"o {eo:.3e}, S_T {es:.3e}"


def test_packed_unsplit_when_short():
    """Sequences no longer than 32 chunks are never split; a packed batch of
    them still matches."""
    lens = [2048, 1, 2047, 0, 1500]
    assert max(packed_plan(lens, 4, cus())) == 1
    wl = I.make_forward(1, sum(lens), 4, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0,
                        s0_std=0.1, seqlens=lens, seed=142)
    check_packed(wl, "packed, no sequence split")
