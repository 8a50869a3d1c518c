"""The workspace is scratch: its contents on entry do not matter (include/gdr2.h,
gdr2_chunk_fwd_workspace_bytes and gdr2_chunk_bwd_workspace_bytes).  Needs an MI355X.

Every kernel writes each workspace value it later reads within the same call,
including the per-chunk flags that send strongly decaying chunks to the
exact-decay launches.  A packed call leaves spare chunk slots (the workspace
is sized for ceil(T/64) + num_seqs chunks) whose flags no kernel of that call
writes; the launches that read them must skip them.  These tests run the same
packed, partly strongly decaying calls on a workspace filled with zero bytes
and on one filled with 0xFF bytes (every flag set, every float a NaN), and
require bitwise-equal results, which also holds the calls to being
deterministic.
"""
import pytest
import torch

import gdr2_inputs as I

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LENS = [70, 0, 129, 5, 200, 64]  # 468 tokens: 9 chunk slots used of ceil(468/64) + 6 = 14


def G():
    import linear_attention_sequence_gdr_amd as g
    return g


def workload(dtype, seed):
    wl = I.make_forward(1, sum(LENS), 3, 128, 64, dtype=dtype, la_dtype=torch.float32,
                        decay_shift=-2.0, s0_std=0.1, seqlens=LENS, seed=seed)
    # about 1% of the log-decay entries at -60: some chunks take the exact path
    gen = torch.Generator("cpu").manual_seed(seed + 1)
    la = wl.log_alpha.float()
    pick = torch.rand(la.shape, generator=gen) < 0.01
    wl.log_alpha = torch.where(pick, torch.full_like(la, -60.0), la).contiguous()
    return wl


def filled(nbytes, byte):
    return torch.full((nbytes,), byte, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_forward_ignores_workspace_contents(dtype):
    wl = workload(dtype, 301)
    ins = [x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    S0, cu = wl.S0.cuda(), wl.cu_seqlens.cuda()
    n = G().gdr2_chunk_fwd_workspace_bytes(1, sum(LENS), 3, 128, 64, len(LENS),
                                           G().GDR2_BF16 if dtype == torch.bfloat16 else G().GDR2_F32)
    outs = []
    for byte in (0x00, 0xFF, 0x00):
        o, ST = G().gdr2_chunk_fwd(*ins, S0, cu, workspace=filled(n, byte))
        torch.cuda.synchronize()
        outs.append((o.cpu(), ST.cpu()))
    for o, ST in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(ST, outs[0][1])
    assert torch.isfinite(outs[0][0].float()).all() and torch.isfinite(outs[0][1]).all()


def test_backward_ignores_workspace_contents():
    wl = workload(torch.bfloat16, 303)
    dO, dST = I.cotangents(wl, seed=304)
    ins = [x.cuda() for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    n = G().gdr2_chunk_bwd_workspace_bytes(1, sum(LENS), 3, 128, 64, len(LENS))
    outs = []
    for byte in (0x00, 0xFF, 0x00):
        g = G().gdr2_chunk_bwd(*ins, dO.cuda(), wl.S0.cuda(), dST.cuda(), wl.cu_seqlens.cuda(),
                               workspace=filled(n, byte))
        torch.cuda.synchronize()
        outs.append({k: v.cpu() for k, v in g.items() if v is not None})
    for g in outs[1:]:
        for k, v in g.items():
            assert torch.equal(v, outs[0][k]), k
    for k, v in outs[0].items():
        assert torch.isfinite(v).all(), k
