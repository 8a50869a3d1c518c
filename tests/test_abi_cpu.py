"""C-ABI contract of libgdr2 on the CPU: the library loads with no GPU present,
exports every entry point include/gdr2.h declares, and rejects bad arguments on
the host before any device call (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import linear_attention_sequence_gdr_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr2.h")
A = 0x10000            # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10008          # misaligned

pytestmark = pytest.mark.skipif(not os.path.exists(G.library_path), reason="libgdr2.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr2_[a-z_0-9]+)\s*\(", src)))


def test_header_and_exports_agree():
    decl = declared_functions()
    assert set(decl) == set(G.EXPORTS), decl
    out = subprocess.run(["nm", "-D", "--defined-only", G.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdr2_[a-z_0-9]+)$", out, flags=re.M))
    missing = set(decl) - exported
    assert not missing, f"declared but not exported: {missing}"
    lib = G.library()
    for name in decl:
        assert hasattr(lib, name)


def test_version_and_strings():
    assert G.gdr2_version() >= 100
    for s in range(8):
        assert G.gdr2_status_string(s)


def fwd(**kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, o=A, ST=None, cu=None, ns=0, B=2, T=100,
                H=4, dk=128, dv=128, dt=G.GDR2_BF16, ldt=G.GDR2_BF16, ws=None, wsb=0, stream=None)
    args.update(kw)
    return G.library().gdr2_chunk_fwd(*args.values())


def dec(**kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S=A, o=A, N=8, H=4, dk=128, dv=128,
                dt=G.GDR2_F32, ldt=G.GDR2_F32, stream=None)
    args.update(kw)
    return G.library().gdr2_decode_step(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(la=None), 1),
    (dict(dt=7), 3), (dict(ldt=-1), 3),
    (dict(B=0), 2), (dict(T=-1), 2), (dict(H=0), 2), (dict(dk=0), 2),
    (dict(dk=48), 5), (dict(dv=256), 5), (dict(dt=G.GDR2_F32, dk=128), 6),
    (dict(cu=A, ns=3), 2), (dict(cu=A, B=1, ns=0), 2),
    (dict(q=MIS), 4), (dict(S0=MIS), 4), (dict(cu=MIS, B=1, ns=3), 4),
    (dict(cu=A, B=1, ns=3), 6), (dict(cu=A, B=1, ns=3, ws=A, wsb=8), 6),
])
def test_chunk_fwd_rejects(kw, status):
    assert fwd(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_chunk_fwd")


@pytest.mark.parametrize("kw,status", [
    (dict(S=None), 1), (dict(q=None), 1), (dict(dt=5), 3), (dict(N=-1), 2), (dict(H=0), 2),
    (dict(dk=16), 5), (dict(o=MIS), 4), (dict(S=MIS), 4),
])
def test_decode_rejects(kw, status):
    assert dec(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_decode_step")


def test_workspace_query():
    q = G.gdr2_chunk_fwd_workspace_bytes
    a256 = lambda x: (x + 255) // 256 * 256
    # fp32 inputs: the fp32 blocks of the backward's front pass, per (chunk, head)
    # (include/gdr2.h: gdr2_chunk_bwd_workspace_bytes), plus packed-sequence tables,
    # then from the next 256-byte boundary one int per item (its exact-decay flag)
    qb = G.gdr2_chunk_bwd_workspace_bytes
    for dk, dv in ((64, 64), (128, 128), (32, 128)):
        item = a256((4 * 64 * dk + 3 * 64 * dv + 2 * 64 * 64 + 2 * dk * dv + dk) * 4)
        assert q(1, 100, 16, dk, dv, 0, G.GDR2_F32) == qb(1, 100, 16, dk, dv, 0) == \
            2 * 16 * item + 2 * 16 * 4
        assert q(2, 300, 3, dk, dv, 0, G.GDR2_F32) == 2 * 5 * 3 * item + 2 * 5 * 3 * 4
        assert q(1, 100, 16, dk, dv, 64, G.GDR2_F32) == qb(1, 100, 16, dk, dv, 64) == \
            a256(65 * 4) + a256(66 * 8) + 66 * 16 * item + 66 * 16 * 4
    # 16-bit inputs: one record per (chunk, head), plus the packed-sequence tables
    # record of the intra-chunk pass (include/gdr2.h): fp16 fragments -Y and Q_g
    # (4*dk/32 KiB each), K_tail (2*dk/16 KiB), A_qk (6 KiB), U (dv/16*4 tiles of
    # 512 B) and fp32 gamma_C (4*dk B)
    def rec_bytes(dk, dv):
        return 2 * 4 * (dk // 32) * 1024 + 2 * (dk // 16) * 1024 + 6 * 1024 + (dv // 16) * 4 * 512 + 4 * dk
    rec = rec_bytes(128, 128)
    # then, from the next 256-byte boundary, one int per record: its chunk took
    # the exact-decay path
    fl = lambda before, recs: a256(before) + recs * 4
    assert q(4, 4096, 16, 128, 128, 0, G.GDR2_BF16) == fl(4 * 64 * 16 * rec, 4 * 64 * 16)
    assert q(1, 100, 16, 128, 128, 0, G.GDR2_BF16) == fl(2 * 16 * rec, 2 * 16)
    cap = 2 + 64
    assert q(1, 100, 16, 128, 128, 64, G.GDR2_BF16) == \
        fl(a256(64 * 4) + a256(65 * 4) + a256(cap * 8) + cap * 16 * rec, cap * 16)
    assert q(2, 64, 3, 32, 64, 0, G.GDR2_BF16) == fl(2 * 1 * 3 * rec_bytes(32, 64), 2 * 3)
    # few long chains: P segments per sequence add transfer matrices and end states
    # (B*P*H*dk*(dk+dv) fp32 from the next 256-byte boundary)
    assert q(1, 32768, 16, 128, 128, 0, G.GDR2_BF16) == \
        fl(a256(512 * 16 * rec) + 16 * 16 * 128 * 256 * 4, 512 * 16)
    assert q(1, 32768, 32, 128, 128, 0, G.GDR2_BF16) == \
        fl(a256(512 * 32 * rec) + 8 * 32 * 128 * 256 * 4, 512 * 32)
    assert q(1, 32768, 1, 64, 64, 0, G.GDR2_BF16) == \
        fl(a256(512 * rec_bytes(64, 64)) + 16 * 64 * 128 * 4, 512)
    # 1000 chunks, 16 segments of 63 chunks (the last 55)
    assert q(2, 64000, 4, 32, 32, 0, G.GDR2_BF16) == \
        fl(a256(2 * 1000 * 4 * rec_bytes(32, 32)) + 2 * 16 * 4 * 32 * 64 * 4, 2 * 1000 * 4)
    # packed sequences with dk == dv and more than 32 chunks in all may be split
    # by the plan built on the device: after the chunk table come the plan (4
    # ints per segment, 2 per sequence, then 256 B for the count) for at most
    # nsmax = N + cap // 32 segments, and after the records the transfer
    # matrices and end states of nsmax * H (segment, head) chains
    def packed(T, N, H, d):
        cap = (T + 63) // 64 + N
        nsmax = N + cap // 32
        head = (a256(N * 4) if 1 < N <= 4096 else 0) + a256((N + 1) * 4) + a256(cap * 8)
        head += a256(nsmax * 16) + a256(N * 8) + 256
        recs = head + cap * H * rec_bytes(d, d)
        return fl(a256(recs) + nsmax * H * d * 2 * d * 4, cap * H)
    assert q(1, 32768 + 63 * 256, 16, 128, 128, 64, G.GDR2_BF16) == packed(32768 + 63 * 256, 64, 16, 128)
    assert q(1, 267139, 16, 128, 128, 64, G.GDR2_BF16) == packed(267139, 64, 16, 128)
    assert q(1, 5000, 3, 32, 32, 1, G.GDR2_BF16) == packed(5000, 1, 3, 32)
    # 32 chunks or fewer in all: never split, no plan
    cap = 32 + 5
    assert q(1, 2048, 4, 128, 128, 5, G.GDR2_BF16) == \
        fl(a256(5 * 4) + a256(6 * 4) + a256(cap * 8) + cap * 4 * rec, cap * 4)
    # dk != dv: never split
    cap = 80 + 3
    assert q(1, 80 * 64, 2, 64, 128, 3, G.GDR2_BF16) == \
        fl(a256(3 * 4) + a256(4 * 4) + a256(cap * 8) + cap * 2 * rec_bytes(64, 128), cap * 2)
    # no split: enough chains, too short, dk != dv
    assert q(4, 32768, 16, 128, 128, 0, G.GDR2_BF16) == fl(4 * 512 * 16 * rec, 4 * 512 * 16)
    assert q(1, 1024, 16, 128, 128, 0, G.GDR2_BF16) == fl(16 * 16 * rec, 16 * 16)
    assert q(1, 32768, 16, 64, 128, 0, G.GDR2_BF16) == fl(512 * 16 * rec_bytes(64, 128), 512 * 16)
    assert q(1, 100, 16, 48, 128, 64, G.GDR2_BF16) == 0
    assert q(0, 100, 16, 128, 128, 64, G.GDR2_BF16) == 0


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 8, 2, 32)
    with pytest.raises(ValueError, match="GPU tensor"):
        G.gdr2_chunk_fwd(x, x, x, x, x, x, o=torch.zeros(1, 8, 2, 32), S_T=torch.zeros(1, 2, 32, 32))
    with pytest.raises(ValueError, match="GPU tensor"):
        y = torch.zeros(4, 2, 32)
        G.gdr2_decode_step(y, y, y, y, y, y, torch.zeros(4, 2, 32, 32), o=torch.zeros(4, 2, 32))


def test_binding_has_no_fallback(monkeypatch):
    monkeypatch.setattr(G, "library_path", "/nonexistent/libgdr2.so")
    monkeypatch.setattr(G, "_lib", None)
    with pytest.raises(G.LibraryMissing):
        G.library()


def ng(**kw):
    args = dict(o=A, z=A, wt=None, y=A, rows=64, d=128, group=128, eps=1e-6, dt=G.GDR2_BF16,
                stream=None)
    args.update(kw)
    return G.library().gdr2_norm_gate(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(z=None), 1), (dict(y=None), 1), (dict(dt=4), 3),
    (dict(rows=-1), 2), (dict(d=0), 2), (dict(group=0), 2), (dict(group=12, d=24), 2),
    (dict(group=64, d=96), 2), (dict(group=16384, d=16384), 2), (dict(eps=-1.0), 2),
    (dict(eps=float("inf")), 2), (dict(eps=float("nan")), 2), (dict(rows=1 << 60), 2),
    (dict(o=MIS), 4), (dict(wt=MIS), 4), (dict(y=MIS), 4),
])
def test_norm_gate_rejects(kw, status):
    assert ng(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_norm_gate")


def test_norm_gate_empty_is_a_no_op():
    # rows = 0 launches nothing, so fake device addresses are never touched
    assert ng(rows=0) == 0
    assert ng(rows=0, o=None, z=None, y=None) == 0


def decg(**kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S=A, z=A, nw=None, eps=1e-6, y=A, N=8, H=4,
                dk=128, dv=128, dt=G.GDR2_BF16, ldt=G.GDR2_F32, stream=None)
    args.update(kw)
    return G.library().gdr2_decode_step_norm_gate(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), 1), (dict(y=None), 1), (dict(S=None), 1), (dict(dt=3), 3), (dict(N=-1), 2),
    (dict(eps=-0.5), 2), (dict(eps=float("nan")), 2), (dict(dv=96), 5),
    (dict(z=MIS), 4), (dict(nw=MIS), 4), (dict(y=MIS), 4),
])
def test_decode_norm_gate_rejects(kw, status):
    assert decg(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_decode_step_norm_gate")


def blk(**kw):
    args = dict(q=A, k=A, v=A, f=A, b=A, w=A, da=A, db=A, flags=7, bs=1.0, eps=1e-6, S0=None, o=A,
                ST=None, cu=None, ns=0, B=2, T=100, H=4, Hv=8, dk=128, dv=128, fdt=G.GDR2_F32,
                ws=None, wsb=0, stream=None)
    args.update(kw)
    return G.library().gdr2_chunk_fwd_block(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(f=None), 1), (dict(da=None), 1), (dict(db=None), 1),
    (dict(fdt=9), 3), (dict(flags=8), 5), (dict(flags=0x17), 5),
    (dict(Hv=6), 2), (dict(Hv=0), 2), (dict(H=0), 2), (dict(T=-1), 2),
    (dict(dk=96), 5), (dict(dv=16), 5),
    (dict(bs=float("inf")), 2), (dict(eps=-1e-6), 2), (dict(eps=float("nan")), 2),
    (dict(cu=A, ns=2), 2), (dict(cu=A, B=1, ns=0), 2),
    (dict(q=MIS), 4), (dict(da=MIS), 4), (dict(db=MIS), 4), (dict(o=MIS), 4),
    (dict(), 6), (dict(ws=A, wsb=1024), 6),
])
def test_chunk_fwd_block_rejects(kw, status):
    assert blk(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_chunk_fwd_block")


def test_chunk_fwd_block_optional_arguments():
    # without GDR2_PRO_DECAY the decay parameters may be NULL; without the gates
    # an infinite b_scale is ignored; both still need the workspace (status 6)
    assert blk(da=None, db=None, flags=5) == 6
    assert blk(flags=3, bs=float("inf")) == 6
    assert blk(flags=6, eps=-1.0) == 6


def bwdc(**kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, dO=A, dST=None, dq=A, dk=A, dv=A, dg=A,
                db=A, dw=A, dS0=None, cu=None, ns=0, B=2, T=100, H=4, dk_=128, dv_=128,
                dt=G.GDR2_BF16, ldt=G.GDR2_F32, ws=None, wsb=0, stream=None)
    args.update(kw)
    return G.library().gdr2_chunk_bwd(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(dO=None), 1), (dict(dg=None), 1), (dict(q=None), 1), (dict(dt=2), 3),
    (dict(B=0), 2), (dict(T=-1), 2), (dict(dk_=48), 5), (dict(dv_=256), 5),
    (dict(cu=A, ns=3), 2), (dict(cu=A, B=1, ns=0), 2),
    (dict(dO=MIS), 4), (dict(dS0=MIS), 4), (dict(dST=MIS), 4),
    (dict(), 6), (dict(ws=A, wsb=4096), 6),
])
def test_chunk_bwd_rejects(kw, status):
    assert bwdc(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_chunk_bwd")


def test_chunk_bwd_workspace_query():
    q = G.gdr2_chunk_bwd_workspace_bytes
    item = lambda dk, dv: (4 * 64 * dk + 3 * 64 * dv + 2 * 64 * 64 + 2 * dk * dv + dk + 63) // 64 * 64 * 4
    a256 = lambda x: (x + 255) // 256 * 256
    # the fp32 blocks, then from the next 256-byte boundary one int per item
    assert q(4, 4096, 16, 128, 128, 0) == 4 * 64 * 16 * item(128, 128) + 4 * 64 * 16 * 4
    assert q(2, 100, 3, 64, 32, 0) == 2 * 2 * 3 * item(64, 32) + 2 * 2 * 3 * 4
    assert q(1, 100, 2, 32, 32, 5) == a256(6 * 4) + a256(2 * 4 * 7) + 7 * 2 * item(32, 32) + 7 * 2 * 4
    assert q(1, 100, 2, 48, 32, 0) == 0


def noalloc(**kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, o=A, ST=None, cu=None, ns=0, B=2, T=100,
                H=4, dk=128, dv=128, dt=G.GDR2_BF16, ldt=G.GDR2_BF16, stream=None)
    args.update(kw)
    return G.library().gdr2_chunk_fwd_noalloc(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(dt=7), 3), (dict(B=0), 2), (dict(dk=48), 5), (dict(q=MIS), 4),
    (dict(cu=A, ns=3), 2),
    # B4 T4096 H16 d128 needs about 296 MB of workspace, more than the 256 MiB scratch
    (dict(B=4, T=4096, H=16), 6),
    (dict(B=1, T=64 * 1200, H=16, dt=G.GDR2_F32, ldt=G.GDR2_F32), 6),
])
def test_noalloc_rejects_on_the_host(kw, status):
    """Argument errors, and sizes whose workspace exceeds the static scratch,
    are refused before any device call (no GPU here)."""
    assert noalloc(**kw) == status
    assert G.gdr2_last_error().startswith("gdr2_chunk_fwd_noalloc")


def test_noalloc_limit_matches_the_workspace_query():
    q = G.gdr2_chunk_fwd_workspace_bytes
    assert q(3, 4096, 16, 128, 128, 0, G.GDR2_BF16) <= G.NOALLOC_SCRATCH_BYTES
    assert q(4, 4096, 16, 128, 128, 0, G.GDR2_BF16) > G.NOALLOC_SCRATCH_BYTES
    hdr = open(HEADER).read()
    assert "#define GDR2_NOALLOC_SCRATCH_BYTES (256u << 20)" in hdr
    assert G.NOALLOC_SCRATCH_BYTES == 256 << 20
