"""The forward and the decode step captured in a HIP graph and replayed
(needs an MI355X).

A caller that captures a graph cannot allocate inside it; the forward with
its outputs and workspace passed in, and the allocation-free forward, enqueue
kernel launches only (no memset, no allocation, no host synchronisation), so
a captured call replays like the eager one.  Each case captures once, then
between replays changes the inputs in place with ordinary eager work, replays,
waits, and checks the replay against an eager call on the same inputs, bit
for bit (the kernels are deterministic).  The first replay is also held to
the parity bar against the fp64 oracle.
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


def capture(fn):
    """Warm fn up on a side stream (as graph capture requires), then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("noalloc,packed", [(True, False), (True, True), (False, True)])
def test_forward_graph_replays(noalloc, packed):
    if packed:
        lens = [3000, 5, 0, 700, 9000, 64]
        wl = I.make_forward(1, sum(lens), 2, 128, 128, decay_shift=-2.0, s0_std=0.1, seqlens=lens, seed=160)
    else:
        wl = I.make_forward(2, 700, 4, 128, 128, decay_shift=-2.0, s0_std=0.1, seed=161)
    q, k, v, la, b, w = (x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w))
    S0 = wl.S0.cuda()
    cu = None if wl.cu_seqlens is None else wl.cu_seqlens.cuda()
    o = torch.empty_like(v)
    ST = torch.empty_like(S0)
    ws = None if noalloc else torch.empty(
        G().gdr2_chunk_fwd_workspace_bytes(wl.B, wl.T, wl.H, 128, 128, wl.num_seqs if packed else 0,
                                           G().GDR2_BF16), dtype=torch.uint8, device="cuda")

    def fwd(out, st):
        if noalloc:
            G().gdr2_chunk_fwd_noalloc(q, k, v, la, b, w, S0, cu, out, st)
        else:
            G().gdr2_chunk_fwd(q, k, v, la, b, w, S0, cu, o=out, S_T=st, workspace=ws)

    g = capture(lambda: fwd(o, ST))
    gen = torch.Generator("cpu").manual_seed(162)
    o2, ST2 = torch.empty_like(o), torch.empty_like(ST)
    for rep in range(4):
        if rep:
            # eager work between replays: new values and new states in place
            v.copy_(torch.randn(v.shape, generator=gen).to(v.dtype))
            S0.mul_(0.5).add_(0.01)
        g.replay()
        torch.cuda.synchronize()
        got = (o.cpu(), ST.cpu())
        fwd(o2, ST2)
        torch.cuda.synchronize()
        assert torch.equal(got[0], o2.cpu()) and torch.equal(got[1], ST2.cpu()), f"replay {rep}"
        if rep == 0:
            ro, rS = oracle.fwd(wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w, S0=wl.S0,
                                cu_seqlens=None if cu is None else wl.cu_seqlens.numpy())
            eo, es = M.bf16_excess(got[0], ro), M.rms_err(got[1], rS)
            M.record(f"graph replay noalloc={noalloc} packed={packed}", o_beyond_bf16_rounding=eo, S_T=es)
            assert eo <= 2e-2 and es <= 2e-2, f"o {eo:.3e}, S_T {es:.3e}"


def test_decode_graph_replays():
    """One captured decode step replayed 8 times, with the step's inputs
    rewritten in place before each replay, equals 8 eager steps."""
    gen = torch.Generator("cpu").manual_seed(163)
    N, H, D = 16, 4, 128
    draws = []
    for _ in range(8):
        x = [torch.randn(N, H, D, generator=gen) for _ in range(6)]
        x[0] = x[0] / x[0].norm(dim=-1, keepdim=True)
        x[1] = x[1] / x[1].norm(dim=-1, keepdim=True)
        x[3] = -torch.nn.functional.softplus(x[3])
        x[4] = torch.sigmoid(x[4])
        x[5] = torch.sigmoid(x[5])
        draws.append(x)
    S_init = 0.1 * torch.randn(N, H, D, D, generator=gen)
    ins = [x.clone().cuda() for x in draws[0]]
    S = S_init.clone().cuda()
    o = torch.empty(N, H, D, device="cuda")
    g = capture(lambda: G().gdr2_decode_step(*ins, S, o=o))
    # the warm-up and the capture's own run stepped S: start again
    S.copy_(S_init.cuda())
    S_e = S_init.clone().cuda()
    for t in range(8):
        for dst, src in zip(ins, draws[t]):
            dst.copy_(src.cuda())
        g.replay()
        o_e = G().gdr2_decode_step(*[x.cuda() for x in draws[t]], S_e)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), o_e.cpu()), f"step {t}: o"
    assert torch.equal(S.cpu(), S_e.cpu())
