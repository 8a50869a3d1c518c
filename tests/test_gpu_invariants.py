"""Structural invariants of the GPU path (needs an MI355X), the pages' facts
that hold at any size, checked through the C ABI:

- decode applied T times equals the chunkwise forward (both run Eq. 10 of the
  pages' "The Gated Delta Rule-2 State Update": the chunkwise form is an exact
  reformulation of the same recurrence);
- the output and end state are linear in (S0, v) jointly for fixed q, k,
  log_alpha, b, w (Eq. 10 is linear in S and in z = w * v): superposition on
  the fp32 path, and homogeneity under a power-of-two scale on the bf16 path,
  where every product and rounding scales with it (up to fp16 subnormals);
- the value channels are independent columns of the recurrence, so permuting
  them (in v, w and S0) permutes the columns of o and S_T; permuting the key
  channels (in q, k, log_alpha, b and the rows of S0) leaves o unchanged and
  permutes the rows of S_T.

Tolerances: fp32 max relative error <= 1e-4, bf16 max-abs / RMS <= 2e-2
(tests/metrics.py), or bitwise where the arithmetic is the same.
"""
import numpy as np
import pytest
import torch

import gdr2_inputs as I
from tests import metrics as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def dev(x):
    return None if x is None else x.cuda()


def fwd(q, k, v, la, b, w, S0, **kw):
    o, ST = G().gdr2_chunk_fwd(dev(q), dev(k), dev(v), dev(la), dev(b), dev(w), dev(S0), None, **kw)
    torch.cuda.synchronize()
    return o.cpu(), ST.cpu()


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 64, 64), (torch.float32, 32, 128),
                                         (torch.bfloat16, 128, 128)])
def test_decode_steps_equal_chunk_forward(dtype, dk, dv):
    """T decode steps from S0 give the forward's o at every token and its S_T
    (the state kept in fp32 between steps, o of each step in the input dtype)."""
    B, T, H = 2, 150, 3
    wl = I.make_forward(B, T, H, dk, dv, dtype=dtype, decay_shift=-2.0, s0_std=0.1, seed=90)
    o, ST = fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, wl.S0)
    S = dev(wl.S0).clone()
    od = torch.empty((B, T, H, dv), dtype=dtype)
    for t in range(T):
        x = [dev(z[:, t].contiguous()) for z in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
        od[:, t] = G().gdr2_decode_step(*x, S).cpu()
    torch.cuda.synchronize()
    S = S.cpu()
    if dtype == torch.float32:
        assert M.max_rel(od, o) <= 1e-4 and M.max_rel(S, ST) <= 1e-4
    else:
        # both outputs are stored in bf16: beyond the two storage roundings
        # (one bf16 step in all), the bf16 bar on the difference
        a, r = M.as64(od.float()), M.as64(o.float())
        excess = np.maximum(np.abs(a - r) - 2 * M.bf16_half_ulp(r), 0.0).max() / M.rms(r)
        assert excess <= 2e-2 and M.rms_err(S, ST) <= 2e-2


def test_superposition_fp32():
    """f(S0a + S0b, va + vb) = f(S0a, va) + f(S0b, vb) with q, k, log_alpha, b,
    w shared (fp32 path, 200 tokens over four chunks)."""
    B, T, H, d = 2, 200, 2, 64
    a = I.make_forward(B, T, H, d, d, dtype=torch.float32, s0_std=0.1, seed=91)
    bb = I.make_forward(B, T, H, d, d, dtype=torch.float32, s0_std=0.1, seed=92)
    oa, Sa = fwd(a.q, a.k, a.v, a.log_alpha, a.b, a.w, a.S0)
    ob, Sb = fwd(a.q, a.k, bb.v, a.log_alpha, a.b, a.w, bb.S0)
    os_, Ss = fwd(a.q, a.k, a.v + bb.v, a.log_alpha, a.b, a.w, a.S0 + bb.S0)
    assert M.max_rel(os_, oa + ob) <= 1e-4 and M.max_rel(Ss, Sa + Sb) <= 1e-4


@pytest.mark.parametrize("split", [False, True])
def test_homogeneity_bf16(split):
    """Scaling S0 and v by 2 scales o and S_T by 2 on the bf16 path.  Every
    operand the scale reaches changes by a power of two, so every rounding does
    too, except where an fp16 operand copy falls among the subnormals (below
    2^-14), where round(2x) may differ from 2 round(x) by 2^-24.  Hence S_T
    within 1e-5 of its RMS and o within one bf16 rounding of 2 o.  With
    split=True the state pass is split into segments (transfer pass and scan)."""
    B, T, H, d = (1, 4096, 2, 128) if split else (2, 333, 4, 128)
    wl = I.make_forward(B, T, H, d, d, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1, seed=93)
    o1, S1 = fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, wl.S0)
    o2, S2 = fwd(wl.q, wl.k, wl.v * 2, wl.log_alpha, wl.b, wl.w, wl.S0 * 2)
    assert M.rms_err(S2, S1 * 2) <= 1e-5
    ulp = torch.abs(o1.float() * 2) * 2.0 ** -7 + 1e-30  # one bf16 step at the value's scale
    assert bool(((o2.float() - o1.float() * 2).abs() <= ulp).all())


def test_value_channel_permutation_bitwise():
    """Permuting the value channels of v, w and S0 permutes the columns of o
    and S_T, bit for bit: every value channel runs the same arithmetic."""
    B, T, H, dk, dv = 2, 200, 4, 128, 128
    wl = I.make_forward(B, T, H, dk, dv, dtype=torch.bfloat16, decay_shift=-2.0, s0_std=0.1, seed=94)
    perm = torch.randperm(dv, generator=torch.Generator().manual_seed(5))
    o1, S1 = fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, wl.S0)
    o2, S2 = fwd(wl.q, wl.k, wl.v[..., perm].contiguous(), wl.log_alpha, wl.b,
                 wl.w[..., perm].contiguous(), wl.S0[..., perm].contiguous())
    assert torch.equal(o2, o1[..., perm]) and torch.equal(S2, S1[..., perm])


def test_key_channel_permutation():
    """Permuting the key channels of q, k, log_alpha, b and the rows of S0
    leaves o unchanged and permutes the rows of S_T (to the fp32 bar: the
    products sum the key channels in another order)."""
    B, T, H, d = 2, 200, 2, 64
    wl = I.make_forward(B, T, H, d, d, dtype=torch.float32, decay_shift=-2.0, s0_std=0.1, seed=95)
    perm = torch.randperm(d, generator=torch.Generator().manual_seed(6))
    o1, S1 = fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, wl.S0)
    p = lambda x: x[..., perm].contiguous()
    o2, S2 = fwd(p(wl.q), p(wl.k), wl.v, p(wl.log_alpha), p(wl.b), wl.w, wl.S0[:, :, perm].contiguous())
    assert M.max_rel(o2, o1) <= 1e-4 and M.max_rel(S2, S1[:, :, perm]) <= 1e-4
