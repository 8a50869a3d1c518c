"""Large values and states on the GPU path (needs an MI355X).

The 16-bit path multiplies the state, the chunk's write targets U = A (w * v)
and the residuals R = U - Y S as fp16 operands, so it is exact to its bar only
while those stay inside the fp16 range (|x| < 65504, stated in
include/gdr2.h); beyond it o and S_T come out non-finite, which this file
shows.  The fp32 path takes fp32 operands and has no such bound: at the same
magnitudes it meets the 1e-4 bar against the fp64 oracle (Gated DeltaNet-2
pages, "The Gated Delta Rule-2 State Update", Eq. 10: the recurrence is linear
in (S0, v), so the scale itself carries no information the oracle lacks).
"""
import pytest
import torch

import gdr2_inputs as I
import oracle
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def run(wl):
    dev = lambda x: None if x is None else x.cuda()
    o, ST = G().gdr2_chunk_fwd(*(dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)),
                               dev(wl.S0), dev(wl.cu_seqlens))
    torch.cuda.synchronize()
    return o.cpu(), ST.cpu()


def scaled(dtype, s0_scale, v_scale, seed):
    wl = I.make_forward(1, 130, 2, 128, 128, dtype=dtype, la_dtype=torch.float32,
                        decay_shift=-2.0, s0_std=0.1, seed=seed)
    wl.S0 = (wl.S0 * s0_scale).contiguous()
    wl.v = (wl.v.float() * v_scale).to(dtype).contiguous()
    return wl


@pytest.mark.parametrize("s0_scale,v_scale", [(1e4, 1.0), (1.0, 1e3)])
def test_bf16_inside_fp16_range(s0_scale, v_scale):
    """max |S0| about 5e3, or |v| up to about 5e3: inside the bound, the usual bar."""
    wl = scaled(torch.bfloat16, s0_scale, v_scale, seed=120)
    o, ST = run(wl)
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    eo, es = M.bf16_excess(o, ro), M.rms_err(ST, rS)
    M.record(f"bf16 magnitude S0 x{s0_scale:g} v x{v_scale:g}", o=eo, S_T=es)
    assert eo <= 2e-2 and es <= 2e-2, f"o {eo:.3e}, S_T {es:.3e}"


@pytest.mark.parametrize("s0_scale,v_scale", [(2e5, 1.0), (1.0, 1e5)])
def test_bf16_beyond_fp16_range_is_nonfinite(s0_scale, v_scale):
    """|S0| or |v| near 1e5: the documented behaviour, non-finite o and S_T."""
    wl = scaled(torch.bfloat16, s0_scale, v_scale, seed=121)
    assert max(wl.S0.abs().max().item(), wl.v.float().abs().max().item()) > 65520
    o, ST = run(wl)
    assert not torch.isfinite(o.float()).all()
    assert not torch.isfinite(ST).all()


@pytest.mark.parametrize("s0_scale,v_scale", [(2e5, 1.0), (1.0, 1e5), (2e5, 1e5)])
def test_fp32_large_magnitudes(s0_scale, v_scale):
    wl = scaled(torch.float32, s0_scale, v_scale, seed=122)
    o, ST = run(wl)
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0)
    eo, es = M.max_rel(o, ro), M.max_rel(ST, rS)
    M.record(f"fp32 magnitude S0 x{s0_scale:g} v x{v_scale:g}", o=eo, S_T=es)
    assert eo <= 1e-4 and es <= 1e-4, f"o {eo:.3e}, S_T {es:.3e}"
