"""Split chains of the bf16 forward vs the fp64 oracle (needs an MI355X).

With few long (sequence, head) chains and dk == dv, the forward cuts every
sequence's chunks into P segments: a transfer pass forms each segment's
affine map of its entry state (Eq. 23 of the pages' chunkwise form, composed
over the segment), an fp32 scan chains the maps, and the state pass runs all
segments at once.  The segment plan depends on the shape only; `plan` below
restates it so each case states the P it exercises, and the workspace size
the library asks for confirms that plan.  Tolerance as for the rest of the
bf16 path: max-abs error / RMS <= 2e-2 on S_T and on o beyond o's own bf16
storage rounding.
"""
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
    """Two split runs are bitwise equal, and the unsplit state pass (the same
    sequence as one packed sequence, which is never split) agrees to the bf16
    tolerance."""
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
