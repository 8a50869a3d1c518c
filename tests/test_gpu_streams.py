"""Calls on a side stream (needs an MI355X).

Every entry point of the binding takes a `stream`: it enqueues its kernels
there and makes that stream current while it allocates its outputs and
workspace and fills the zeros it needs, so the caching allocator reuses that
memory only in the stream's order.  Each case runs once on the default stream
and once on a side stream (default priority) while the default stream, right
after the side-stream call is enqueued, allocates and fills large buffers of
NaN: a workspace or an output that had been handed back to the default
stream's pool too early would be overwritten by them.  The side-stream
results must equal the default-stream ones bit for bit (the kernels are
deterministic).
"""
import pytest
import torch

import gdr2_inputs as I

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def churn():
    """Allocate and fill 8 x 64 MiB of NaN on the current (default) stream."""
    for _ in range(8):
        x = torch.full((16 << 20,), float("nan"), device="cuda")
        del x


def on_side(fn):
    """Run fn(stream) on a fresh side stream after the default stream's work,
    churn the default stream's pool meanwhile, and wait for the result."""
    cur = torch.cuda.current_stream()
    s = torch.cuda.Stream()
    s.wait_stream(cur)
    out = fn(s)
    churn()
    cur.wait_stream(s)
    torch.cuda.synchronize()
    return out


def same(a, b, what):
    if isinstance(a, dict):
        for k in a:
            same(a[k], b[k], f"{what}[{k}]")
    elif isinstance(a, (tuple, list)):
        for i, (x, y) in enumerate(zip(a, b)):
            same(x, y, f"{what}[{i}]")
    elif a is None:
        assert b is None, what
    else:
        assert torch.equal(a.cpu(), b.cpu()), what


def packed_workload(dtype=torch.bfloat16, dk=64, seed=150):
    lens = [300, 0, 2500, 77, 64]
    return I.make_forward(1, sum(lens), 2, dk, dk, dtype=dtype, la_dtype=torch.float32,
                          decay_shift=-2.0, s0_std=0.1, seqlens=lens, seed=seed)


@pytest.mark.parametrize("packed", [False, True])
def test_forward_on_a_side_stream(packed):
    wl = packed_workload() if packed else I.make_forward(2, 700, 2, 128, 128, s0_std=0.1, seed=151)
    args = [x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    S0 = wl.S0.cuda()
    cu = None if wl.cu_seqlens is None else wl.cu_seqlens.cuda()
    ref = G().gdr2_chunk_fwd(*args, S0, cu)
    torch.cuda.synchronize()
    got = on_side(lambda s: G().gdr2_chunk_fwd(*args, S0, cu, stream=s))
    same(got, ref, f"forward packed={packed}")


def test_packed_backward_on_a_side_stream():
    """The packed backward fills its gradients with zeros first (rows outside
    every sequence): that fill runs on the side stream too."""
    wl = packed_workload(dtype=torch.float32, seed=152)
    dO, dST = I.cotangents(wl, seed=153)
    args = [x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    rest = (dO.cuda(), wl.S0.cuda(), dST.cuda(), wl.cu_seqlens.cuda())
    ref = G().gdr2_chunk_bwd(*args, *rest)
    torch.cuda.synchronize()
    got = on_side(lambda s: G().gdr2_chunk_bwd(*args, *rest, stream=s))
    same(got, ref, "packed backward")


def test_block_and_decode_on_a_side_stream():
    bl = I.make_block(1, 400, 2, 4, 64, 64, s0_std=0.1, seed=154)
    bargs = [x.cuda() for x in (bl.q, bl.k, bl.v, bl.f, bl.b, bl.w, bl.a, bl.delta)]
    S0 = bl.S0.cuda()
    ref = G().gdr2_chunk_fwd_block(*bargs, S0=S0)
    torch.cuda.synchronize()
    got = on_side(lambda s: G().gdr2_chunk_fwd_block(*bargs, S0=S0, stream=s))
    same(got, ref, "block forward")
    gen = torch.Generator("cpu").manual_seed(155)
    N, H, D = 8, 2, 64
    dq = [torch.randn(N, H, D, generator=gen) for _ in range(6)]
    dq[3] = -torch.nn.functional.softplus(dq[3])  # log-decay <= 0
    dq = [x.cuda() for x in dq]
    S = (0.1 * torch.randn(N, H, D, D, generator=gen)).cuda()
    S1 = S.clone()
    o_ref = G().gdr2_decode_step(*dq, S1)
    torch.cuda.synchronize()
    S2 = S.clone()
    o_got = on_side(lambda s: G().gdr2_decode_step(*dq, S2, stream=s))
    same((o_got, S2), (o_ref, S1), "decode")
