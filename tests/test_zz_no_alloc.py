"""gdr2_chunk_fwd_noalloc (static scratch, no allocation) against gdr2_chunk_fwd
(caller's workspace), through the C ABI (needs an MI355X).

Two calls in a row share the device's scratch, the second one with a smaller
input, so whatever the first left in the scratch must not leak into the second.
The two entry points run the same kernels on the same inputs, so the outputs
must agree bit for bit (tighter than the parity bar); the first call is also
checked against the fp64 oracle at that bar.
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


def both(wl):
    dev = lambda x: None if x is None else x.cuda()
    args = [dev(x) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    o_ref, S_ref = G().gdr2_chunk_fwd(*args, dev(wl.S0), dev(wl.cu_seqlens))
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    G().gdr2_chunk_fwd_noalloc(*args, dev(wl.S0), dev(wl.cu_seqlens), o, S)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu(), o_ref.cpu(), S_ref.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_two_calls_second_smaller(dtype):
    big = I.make_forward(2, 1000, 16, 128, 128, dtype=dtype, decay_shift=-2.0, s0_std=0.1, seed=130)
    o, S, o_ref, S_ref = both(big)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ro, rS = oracle.fwd(big.q, big.k, big.v, big.log_alpha, big.b, big.w, S0=big.S0)
    if dtype == torch.bfloat16:
        assert M.bf16_excess(o, ro) <= 2e-2 and M.rms_err(S, rS) <= 2e-2
    else:
        assert M.max_rel(o, ro) <= 1e-4 and M.max_rel(S, rS) <= 1e-4
    lens = [70, 0, 129, 5]
    small = I.make_forward(1, sum(lens), 4, 64, 64, dtype=dtype, decay_shift=-2.0, s0_std=0.1,
                           seqlens=lens, seed=131)
    o, S, o_ref, S_ref = both(small)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_strong_decay_items_then_plain():
    """A call with strong-decay chunks (flagged in the scratch), then a smaller
    plain call on the same scratch."""
    wl = I.make_forward(1, 300, 8, 128, 128, dtype=torch.bfloat16, la_dtype=torch.float32,
                        decay_shift=-2.0, s0_std=0.1, seed=132)
    wl.log_alpha[:, 100:130] = -60.0
    o, S, o_ref, S_ref = both(wl)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    wl2 = I.make_forward(1, 100, 8, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                         seed=133)
    o, S, o_ref, S_ref = both(wl2)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_packed_split_then_unsplit():
    """Packed sequences whose long member the device plan splits (the plan and
    the segment maps live in the scratch), then a smaller packed call that
    splits nothing, on the same scratch."""
    lens = [7000, 30, 0, 2500]
    wl = I.make_forward(1, sum(lens), 2, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seqlens=lens, seed=135)
    o, S, o_ref, S_ref = both(wl)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0,
                        cu_seqlens=wl.cu_seqlens.numpy())
    assert M.bf16_excess(o, ro) <= 2e-2 and M.rms_err(S, rS) <= 2e-2
    lens = [300, 1, 900]
    wl = I.make_forward(1, sum(lens), 2, 128, 128, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1,
                        seqlens=lens, seed=136)
    o, S, o_ref, S_ref = both(wl)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_noalloc_refuses_oversize_before_any_launch():
    wl = I.make_forward(4, 64, 16, 128, 128, dtype=torch.bfloat16, seed=134)
    x = torch.zeros(4, 4096, 16, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(G().Gdr2Error, match="static scratch"):
        G().gdr2_chunk_fwd_noalloc(x, x, x, x, x, x, None, None, x, None)
    del wl
