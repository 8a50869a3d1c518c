"""Benchmark of the Gated Delta Rule-2 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps D] [--no-cpu]

A step is one gdr2_chunk_fwd over the training-shape workload (B=4, T=4096,
H=16, dk=dv=128, bf16 inputs, fp32 state, S0 = 0): inputs are resident in HBM
before timing starts, W untimed steps run first, then exactly K steps are timed
back to back with HIP events on the launch stream.  The same run also times D
decode steps (256 sequences x 16 heads, fp32 state updated in place) and the
fp64 oracle on a bounded sample of the forward workload on the host cores,
and, outside the step, the block's output epilogue (gdr2_norm_gate over the
forward's o), the decode step with that epilogue fused
(gdr2_decode_step_norm_gate), and the same forward from the block's projections
with the gate prologue fused (gdr2_chunk_fwd_block), and the backward of the
forward (gdr2_chunk_bwd).

Prints one JSON line: tokens/s of the forward (whole job), its TFLOP/s and the
HBM roofline of the forward kernel, the decode HBM GB/s with its own roofline,
and the CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
TRAFFIC_FILE = {"fwd": os.path.join(ROOT, "profiles", "traffic_chunk_fwd_b4_t4096_h16_d128.json"),
                "long": os.path.join(ROOT, "profiles", "traffic_chunk_fwd_b1_t32768_h16_d128.json"),
                "varlen": os.path.join(ROOT, "profiles", "traffic_chunk_fwd_varlen64_h16_d128.json"),
                "packed_long": os.path.join(ROOT, "profiles", "traffic_chunk_fwd_packed_long32k_h16_d128.json")}
MFMA_FILE = {"fwd": os.path.join(ROOT, "profiles", "mfma_chunk_fwd_b4_t4096_h16_d128.json"),
             "long": os.path.join(ROOT, "profiles", "mfma_chunk_fwd_b1_t32768_h16_d128.json")}
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32")
# the kernels of one B4 T4096 H16 d128 bf16 gdr2_chunk_fwd call
FWD_KERNELS = ("intra_kernel<128, 128, true, 0, 0>", "state_kernel<128, 128, 2, 4, false, 1>")


def fwd_algorithmic(B, T, H, dk, dv, in_bytes=2, C=64):
    """Algorithmic bytes and flops of one forward (no S0 read, S_T written).

    Bytes: q, k, log_alpha, b (dk each) and v, w (dv each) read once, o written
    once, S_T written once.  Flops per 64-token chunk and head: T and A_qk
    (triangular), Y and U (triangular), A_qk R, and the three state products
    Q_g S, Y S, K_tail^T R.
    """
    tok = B * T * H
    byts = tok * (4 * dk + 2 * dv) * in_bytes + tok * dv * in_bytes + B * H * dk * dv * 4
    per_chunk = (C * (C - 1) * dk + C * (C + 1) * dk + C * (C - 1) * (dk + dv)
                 + C * (C + 1) * dv + 6 * C * dk * dv)
    flops = per_chunk * tok / C
    return byts, flops


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_gdr_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, *kernel_keys):
    """HBM bytes per launch of one kernel (summed over several kernels that
    one call launches) of a workload ("fwd": the B4 T4096 calls, "long": the
    long sequence), from the rocprofv3 counter runs committed under
    profiles/, only when they were taken on the current kernel sources."""
    try:
        with open(TRAFFIC_FILE[workload]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    total = 0.0
    for key in kernel_keys:
        k = t.get("kernels", {}).get(key)
        if k is None:
            return None
        total += k["fetch_bytes"] + k["write_bytes"]
    return total


def load_call_traffic(workload, once_key, *prefixes):
    """HBM bytes of one call that launches several kernels, some of them many
    times: the traffic of every dispatch of the kernels whose names start with
    one of `prefixes`, over the number of calls (the dispatches of `once_key`,
    a kernel launched once per call)."""
    try:
        with open(TRAFFIC_FILE[workload]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    ks = t.get("kernels", {})
    if once_key not in ks:
        return None
    total = sum((k["fetch_bytes"] + k["write_bytes"]) * k["dispatches"]
                for name, k in ks.items() if name.startswith(prefixes))
    return total / ks[once_key]["dispatches"]


def write_mfma(csv_path, command, workload="fwd"):
    """Per-kernel MFMA use from one rocprofv3 --pmc run of MfmaUtil (MFMA-busy
    cycles over active cycles and SIMDs, in percent) and the MFMA op counters
    (units of 512 flops): the average per dispatch of every libgdr2 kernel."""
    per = {}
    for r in _counter_rows(csv_path):
        name = r["Kernel_Name"]
        if "gdr2::" not in name:
            continue
        key = name.split("gdr2::", 1)[1].replace("(anonymous namespace)::", "").split("(", 1)[0]
        per.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    out = {"source_hash": source_hash(), "command": command, "kernels": {}}
    for key, d in per.items():
        util = d.get("MfmaUtil", [0.0])
        flops = {c: sum(d.get(c, [0.0])) / max(1, len(d.get(c, []))) * 512 for c in MFMA_COUNTERS}
        out["kernels"][key] = {"mfma_util_pct": sum(util) / len(util), "dispatches": len(util),
                               "mfma_flops": sum(flops.values()),
                               "mfma_flops_by_type": {c.rsplit("_", 1)[1]: v for c, v in flops.items()}}
    with open(MFMA_FILE[workload], "w") as fo:
        json.dump(out, fo, indent=1)
    print(json.dumps(out))


def load_mfma(workload, *kernel_keys):
    """MFMA-busy percent per kernel and the MFMA flops one call issues (summed
    over kernel_keys), from the committed counter run, only when it was taken
    on the current kernel sources."""
    try:
        with open(MFMA_FILE[workload]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    ks = t.get("kernels", {})
    if any(k not in ks for k in kernel_keys):
        return None
    return {"util_pct": {k: ks[k]["mfma_util_pct"] for k in kernel_keys},
            "issued_flops": sum(ks[k]["mfma_flops"] for k in kernel_keys)}


def _counter_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def write_traffic(fetch_csv, write_csv, copy_mib, command, workload="fwd"):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) into HBM bytes per launch for every libgdr2 kernel.  Each counter
    is scaled by what it reads for the calibration copy (torch.neg over
    copy_mib MiB of fp32: copy_mib MiB read and copy_mib MiB written)."""
    known = copy_mib * 1024 * 1024
    out = {"source_hash": source_hash(), "command": command, "kernels": {}, "calibration": {}}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _counter_rows(path) if r.get("Counter_Name") == counter]
        calib = [float(r["Counter_Value"]) * 1024 for r in rows if "neg" in r["Kernel_Name"]]
        if not calib:
            raise SystemExit(f"{path}: no calibration copy dispatch found")
        factor = max(calib) / known
        out["calibration"][counter] = {"copy_bytes": known, "counter_bytes": max(calib),
                                       "factor": factor}
        for r in rows:
            name = r["Kernel_Name"]
            if "gdr2::" not in name:
                continue
            # the kernel with its template arguments: variants are kept apart
            key = name.split("gdr2::", 1)[1].replace("(anonymous namespace)::", "").split("(", 1)[0]
            per.setdefault(key, {}).setdefault(counter, []).append(
                float(r["Counter_Value"]) * 1024 / factor)
    for key, d in per.items():
        f, w = d.get("FETCH_SIZE", [0.0]), d.get("WRITE_SIZE", [0.0])
        out["kernels"][key] = {"fetch_bytes": sum(f) / len(f), "write_bytes": sum(w) / len(w),
                               "dispatches": len(f)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE[workload]), exist_ok=True)
    with open(TRAFFIC_FILE[workload], "w") as fo:
        json.dump(out, fo, indent=1)
    print(json.dumps(out))


def time_events(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps     # ms per step


def settle(fn, torch, seconds=0.25):
    """Untimed back-to-back calls for about `seconds`: the first milliseconds
    of a process run at lower clocks, which the warm-up steps alone do not
    always cover."""
    import time
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def time_cold(fn, steps, torch, flush_mib=512):
    """Median time of single calls that each follow a write of flush_mib MiB
    of scratch, so the 256 MB last-level cache holds none of the call's
    inputs; the events bracket the call only."""
    scratch = torch.empty(flush_mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    times = []
    for i in range(steps + 1):
        scratch.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        if i:
            times.append(a.elapsed_time(b))
    del scratch
    times.sort()
    return times[len(times) // 2]


def cpu_baseline(wl, budget_s=12.0):
    """The fp64 oracle as it stands, on whole (sequence, head) chains of the
    forward workload, using every host core it is allowed.  The sample is as
    many chains as fit the budget on the cores; when all of them fit, the
    whole workload is repeated until the budget is spent."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    cores = min(cores, oracle.max_threads())  # read before the probe sets the thread count
    N, H = wl.B, wl.H
    # probe one chain to size the sample to the budget
    m = np.zeros((N, H), bool)
    m[0, 0] = True
    q, k, v, g, b, w = (oracle.f64(x[:1]) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w))
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, g, b, w, mask=m[:1], nthreads=1)
    t1 = time.perf_counter() - t0
    pairs = int(max(1, min(N * H, cores * max(1, budget_s // max(t1, 1e-3)))))
    m = np.zeros(N * H, bool)
    m[:pairs] = True
    m = m.reshape(N, H)
    nseq = int(np.ceil(pairs / H))
    q, k, v, g, b, w = (oracle.f64(x[:nseq]) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w))
    used = min(cores, pairs)
    reps, dt = 0, 0.0
    t0 = time.perf_counter()
    while reps == 0 or dt < budget_s:
        oracle.fwd(q, k, v, g, b, w, mask=m[:nseq], nthreads=used)
        reps += 1
        dt = time.perf_counter() - t0
    head_tokens = reps * pairs * wl.T
    return {"value": head_tokens / H / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{reps} x {pairs} of {N * H} (sequence, head) chains x {wl.T} tokens, fp64 "
                      f"token-by-token, {dt:.1f} s on {used} threads; tokens/s counts a token "
                      f"once per {H} heads"}


def long_leg(args, torch, G, I, dev):
    """One long sequence per head: B1 T32768 H16 d128 bf16 with S0, 16 chains of
    512 chunks, each split into 16 segments (transfer pass, fp32 scan, state
    pass)."""
    lw = I.config(3)
    ins = [x.to(dev) for x in (lw.q, lw.k, lw.v, lw.log_alpha, lw.b, lw.w)]
    S0 = lw.S0.to(dev)
    o = torch.empty((lw.B, lw.T, lw.H, lw.dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty_like(S0)
    ws = torch.empty(max(1, G.gdr2_chunk_fwd_workspace_bytes(lw.B, lw.T, lw.H, lw.dk, lw.dv, 0,
                                                             G.GDR2_BF16)),
                     dtype=torch.uint8, device=dev)
    fwd = lambda: G.gdr2_chunk_fwd(*ins, S0, None, o=o, S_T=ST, workspace=ws)
    ms = time_events(fwd, args.steps, args.warmup, torch)
    byts, flops = fwd_algorithmic(lw.B, lw.T, lw.H, lw.dk, lw.dv)
    byts += lw.B * lw.H * lw.dk * lw.dv * 4  # S0 read
    gbs = byts / (ms * 1e-3) / 1e9
    keys = ("intra_kernel<128, 128, true, 0, 0>", "state_kernel<128, 128, 8, 4, true, 2>",
            "scan_kernel<128, 128>", "state_kernel<128, 128, 4, 4, false, 2>")
    mf = load_mfma("long", *keys)
    mfma = None
    if mf:
        issued = mf["issued_flops"] / (ms * 1e-3) / 1e12
        mfma = {"issued_gflop_per_call": mf["issued_flops"] / 1e9, "issued_tflops": issued,
                "issued_frac_of_bf16_peak": issued / BF16_PEAK_TFLOPS, "busy_pct": mf["util_pct"]}
    return {"workload": "gdr2_chunk_fwd B1 T32768 H16 dk=dv=128 bf16, b in [0,2], decay shift -4, "
                        "S0 ~ N(0, 0.1): 16 chains of 512 chunks, each split into 16 segments "
                        "(transfer pass, fp32 scan, state pass)",
            "steps": args.steps, "ms_per_call": ms, "tokens_per_s": lw.B * lw.T / (ms * 1e-3),
            "tflops": flops / (ms * 1e-3) / 1e12, "alg_bytes": byts, "mfma": mfma,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("long", *keys)}}


def ceilings(torch, dev):
    """Measured ceilings beside the published peaks: a copy of 1 GiB into
    another 1 GiB (read and write streams at once), a read-only stream over
    2 GiB (both far beyond the 256 MB last-level cache), and back-to-back
    16x16x32 bf16 and f16 MFMAs from registers on every CU.  Each is the best
    of five launches timed with HIP events on torch's current stream."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "linear_attention_sequence_gdr_amd", "libgdr2_ceiling.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int
    lib.gdr2_ceiling_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.gdr2_ceiling_read.argtypes = [vp, vp, i64, i32, vp]
    lib.gdr2_ceiling_mfma.argtypes = [vp, i32, i32, i32, vp]
    for f in (lib.gdr2_ceiling_copy, lib.gdr2_ceiling_read, lib.gdr2_ceiling_mfma):
        f.restype = i32
    st = torch.cuda.current_stream(dev).cuda_stream

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = fn()
            b.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"ceiling kernel launch failed ({rc})")
            t.append(a.elapsed_time(b))
        return min(t) * 1e-3

    gib = 1 << 30
    src = torch.empty(2 * gib, dtype=torch.uint8, device=dev)
    dst = torch.empty(gib, dtype=torch.uint8, device=dev)
    src.fill_(1)
    red = torch.empty(256 * 64, dtype=torch.int32, device=dev)
    blocks = 256 * 64
    tc = best(lambda: lib.gdr2_ceiling_copy(src.data_ptr(), dst.data_ptr(), gib // 16, blocks, st))
    tr = best(lambda: lib.gdr2_ceiling_read(src.data_ptr(), red.data_ptr(), 2 * gib // 16, blocks, st))
    del src, dst, red
    mb, iters = 256 * 8, 4000
    out = torch.empty(mb * 256, dtype=torch.float32, device=dev)
    flops = mb * 4 * iters * 8 * 16 * 16 * 32 * 2
    tb = best(lambda: lib.gdr2_ceiling_mfma(out.data_ptr(), mb, iters, 0, st))
    th = best(lambda: lib.gdr2_ceiling_mfma(out.data_ptr(), mb, iters, 1, st))
    del out
    return {"hbm_copy_GBs": 2 * gib / tc / 1e9, "hbm_read_GBs": 2 * gib / tr / 1e9,
            "mfma_bf16_TFLOPs": flops / tb / 1e12, "mfma_f16_TFLOPs": flops / th / 1e12,
            "published": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": BF16_PEAK_TFLOPS},
            "method": "copy 1 GiB -> 1 GiB and read 2 GiB with 16-byte vector loads; 16x16x32 "
                      "MFMAs, 8 independent chains per wavefront, 2048 workgroups of 4 "
                      "wavefronts; best of 5, HIP events"}


def cpu_single_thread(wl):
    """The oracle on one (sequence, head) chain of the forward workload on one
    thread: a per-core figure."""
    import numpy as np
    import oracle
    m = np.zeros((1, wl.H), bool)
    m[0, 0] = True
    q, k, v, g, b, w = (oracle.f64(x[:1]) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w))
    oracle.fwd(q[:, :64], k[:, :64], v[:, :64], g[:, :64], b[:, :64], w[:, :64], mask=m, nthreads=1)
    t0 = time.perf_counter()
    oracle.fwd(q, k, v, g, b, w, mask=m, nthreads=1)
    dt = time.perf_counter() - t0
    return {"value": wl.T / dt, "unit": "head-tokens/s", "cores": 1,
            "sample": f"1 (sequence, head) chain x {wl.T} tokens, fp64 token-by-token, {dt:.2f} s"}


def varlen_leg(args, torch, G, I, dev):
    """64 packed sequences of U[1, 8192] tokens (about 262K tokens), H16 d128
    bf16, each with its own S0 and S_T."""
    vw = I.config(4)
    ins = [x.to(dev) for x in (vw.q, vw.k, vw.v, vw.log_alpha, vw.b, vw.w)]
    S0, cu = vw.S0.to(dev), vw.cu_seqlens.to(dev)
    N, T, H, dk, dv = vw.num_seqs, vw.T, vw.H, vw.dk, vw.dv
    o = torch.empty((1, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty_like(S0)
    ws = torch.empty(max(1, G.gdr2_chunk_fwd_workspace_bytes(1, T, H, dk, dv, N, G.GDR2_BF16)),
                     dtype=torch.uint8, device=dev)
    fwd = lambda: G.gdr2_chunk_fwd(*ins, S0, cu, o=o, S_T=ST, workspace=ws)
    steps = max(3, min(args.steps, 10))
    ms = time_events(fwd, steps, 2, torch)
    byts, flops = fwd_algorithmic(1, T, H, dk, dv)
    byts += N * H * dk * dv * 4 - H * dk * dv * 4  # S0 read and N final states (not 1)
    gbs = byts / (ms * 1e-3) / 1e9
    del ins, S0, cu, o, ST, ws
    return {"workload": f"gdr2_chunk_fwd, {N} packed sequences of U[1, 8192] tokens ({T} tokens), "
                        "H16 dk=dv=128 bf16, per-sequence S0 ~ N(0, 0.1), decay shift -2",
            "steps": steps, "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "tflops": flops / (ms * 1e-3) / 1e12, "alg_bytes": byts,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_call_traffic("varlen", "intra_kernel<128, 128, true, 0, 0>",
                                                      "intra_kernel", "state_kernel", "schedule",
                                                      "chunk_table")}}


def packed_long_leg(args, torch, G, I, dev):
    """One 32K-token sequence among 63 short ones, packed: the device plan
    splits the long sequence into segments."""
    vw = I.packed_long()
    ins = [x.to(dev) for x in (vw.q, vw.k, vw.v, vw.log_alpha, vw.b, vw.w)]
    S0, cu = vw.S0.to(dev), vw.cu_seqlens.to(dev)
    N, T, H, dk, dv = vw.num_seqs, vw.T, vw.H, vw.dk, vw.dv
    o = torch.empty((1, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty_like(S0)
    ws = torch.empty(max(1, G.gdr2_chunk_fwd_workspace_bytes(1, T, H, dk, dv, N, G.GDR2_BF16)),
                     dtype=torch.uint8, device=dev)
    fwd = lambda: G.gdr2_chunk_fwd(*ins, S0, cu, o=o, S_T=ST, workspace=ws)
    steps = max(3, min(args.steps, 20))
    ms = time_events(fwd, steps, 2, torch)
    byts, flops = fwd_algorithmic(1, T, H, dk, dv)
    byts += N * H * dk * dv * 4 - H * dk * dv * 4  # S0 read and N final states (not 1)
    gbs = byts / (ms * 1e-3) / 1e9
    del ins, S0, cu, o, ST, ws
    return {"workload": f"gdr2_chunk_fwd, one 32768-token sequence among 63 of U[1, 512] tokens "
                        f"({T} tokens, {N} packed sequences), H16 dk=dv=128 bf16, per-sequence S0 ~ N(0, 0.1), "
                        "decay shift -2; the long sequence is split into segments on the device",
            "steps": steps, "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "tflops": flops / (ms * 1e-3) / 1e12, "alg_bytes": byts,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_call_traffic("packed_long", "intra_kernel<128, 128, true, 0, 0>",
                                                      "intra_kernel", "state_kernel", "scan_kernel",
                                                      "schedule", "chunk_table", "segment_plan")}}


def calibration_copy(args, torch, dev):
    if args.calibrate_copy:
        n = args.calibrate_copy * 1024 * 1024 // 4
        src_t = torch.randn(n, device=dev)
        dst_t = torch.empty_like(src_t)
        for _ in range(3):
            torch.neg(src_t, out=dst_t)
        torch.cuda.synchronize()
        del src_t, dst_t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--varlen", choices=("on", "off", "only"), default="on",
                    help="the packed-sequence forward: in the line (on), left out (off), or alone "
                         "in a line of its own (only; profiling its kernels apart)")
    ap.add_argument("--no-ceilings", action="store_true", help="leave out the measured ceilings")
    ap.add_argument("--no-cold", action="store_true",
                    help="leave out the cold-cache forward timing (keeps kernel-trace averages warm)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain copy of MIB MiB (for counter calibration)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write the per-kernel HBM traffic table from two "
                         "rocprofv3 --pmc counter_collection.csv files")
    ap.add_argument("--traffic-command", default="",
                    help="the command that produced the counter files (recorded)")
    ap.add_argument("--packed-long", choices=("on", "off", "only"), default="on",
                    help="the leg with one 32K-token sequence among 63 short ones (only: that leg alone)")
    ap.add_argument("--traffic-workload", choices=("fwd", "long", "varlen", "packed_long"), default="fwd",
                    help="which workload's kernels the counter files cover")
    ap.add_argument("--mfma", metavar="CSV",
                    help="host only: write the per-kernel MFMA table from a rocprofv3 --pmc "
                         "MfmaUtil + SQ_INSTS_VALU_MFMA_MOPS_* counter_collection.csv")
    ap.add_argument("--long", choices=("on", "off", "only"), default="on",
                    help="the long-sequence forward: in the line (on), left out (off), or "
                         "alone in a line of its own (only; profiling its kernels apart)")
    args = ap.parse_args()
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.calibrate_copy, args.traffic_command,
                      args.traffic_workload)
        return
    if args.mfma:
        write_mfma(args.mfma, args.traffic_command, args.traffic_workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Gated Delta Rule-2 path here has no multi-GPU "
              "mode (sequences and heads shard with no exchange between GPUs). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gdr2_inputs as I
    import linear_attention_sequence_gdr_amd as G

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    G.library()
    if args.long == "only":
        leg = long_leg(args, torch, G, I, dev)
        calibration_copy(args, torch, dev)
        print(json.dumps({"long_sequence": leg, "source_hash": source_hash()}), flush=True)
        return
    if args.varlen == "only":
        leg = varlen_leg(args, torch, G, I, dev)
        calibration_copy(args, torch, dev)
        print(json.dumps({"varlen": leg, "source_hash": source_hash()}), flush=True)
        return
    if args.packed_long == "only":
        leg = packed_long_leg(args, torch, G, I, dev)
        calibration_copy(args, torch, dev)
        print(json.dumps({"packed_long": leg, "source_hash": source_hash()}), flush=True)
        return

    # ---- forward: B4 T4096 H16 d128 bf16 ------------------------------------------------
    wl = I.config(1)
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    ins = [x.to(dev) for x in (wl.q, wl.k, wl.v, wl.log_alpha, wl.b, wl.w)]
    o = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    ws = torch.empty(max(1, G.gdr2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, 0, G.GDR2_BF16)),
                     dtype=torch.uint8, device=dev)
    fwd = lambda: G.gdr2_chunk_fwd(*ins, None, None, o=o, S_T=ST, workspace=ws)
    settle(fwd, torch)
    ms = time_events(fwd, args.steps, args.warmup, torch)
    cold_ms = None if args.no_cold else time_cold(fwd, max(5, min(args.steps, 20)), torch)
    byts, flops = fwd_algorithmic(B, T, H, dk, dv)
    tokens = B * T
    gbs = byts / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    # one gdr2_chunk_fwd call = the intra-chunk pass + the state pass
    traffic = load_traffic("fwd", *FWD_KERNELS)
    mf = load_mfma("fwd", *FWD_KERNELS)
    mfma = None
    if mf:
        issued = mf["issued_flops"] / (ms * 1e-3) / 1e12
        mfma = {"issued_gflop_per_call": mf["issued_flops"] / 1e9, "issued_tflops": issued,
                "issued_frac_of_bf16_peak": issued / BF16_PEAK_TFLOPS,
                "busy_pct": mf["util_pct"],
                "counters": "rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_{F16,BF16,F32}"}

    # ---- the same forward from the block's projections (fused gate prologue) ------
    bl = I.make_block(B, T, H, H, dk, dv, seed=7)
    bargs = [x.to(dev) for x in (bl.q, bl.k, bl.v, bl.f, bl.b, bl.w, bl.a, bl.delta)]
    del bl
    blk = lambda: G.gdr2_chunk_fwd_block(*bargs, flags=7, o=o, S_T=ST, workspace=ws)
    bms = time_events(blk, args.steps, args.warmup, torch)
    bgbs = byts / (bms * 1e-3) / 1e9
    del bargs

    # ---- backward of the same forward (dL/do, dL/dS_T -> every input gradient) ------
    dOb = torch.randn((B, T, H, dv), generator=torch.Generator("cpu").manual_seed(8)).to(torch.bfloat16).to(dev)
    dSTb = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=dev)
    wsb = torch.empty(G.gdr2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, 0), dtype=torch.uint8, device=dev)
    bwd = lambda: G.gdr2_chunk_bwd(*ins, dOb, None, dSTb, workspace=wsb)
    bwd_steps = max(1, min(args.steps, 10))
    settle(bwd, torch, 0.25)
    bwms = time_events(bwd, bwd_steps, 3, torch)
    # algorithmic bytes: q, k, log_alpha, b, v, w, dO read (bf16), dS_T read and dS0
    # written (fp32), six fp32 input gradients written
    bw_bytes = tokens * H * (4 * dk + 3 * dv) * 2 + 2 * B * H * dk * dv * 4 + tokens * H * (4 * dk + 2 * dv) * 4
    bw_gbs = bw_bytes / (bwms * 1e-3) / 1e9
    del dOb, dSTb, wsb

    # ---- decode: 256 sequences x 16 heads, fp32 state ---------------------------------
    S = I.decode_state().to(dev)
    pool = [[t.to(dev) for t in I.decode_step_inputs(s)] for s in range(8)]
    od = torch.empty((I.DECODE_N, I.DECODE_H, I.DECODE_D), dtype=torch.float32, device=dev)
    it = [0]

    def dec():
        x = pool[it[0] % len(pool)]
        it[0] += 1
        G.gdr2_decode_step(*x, S, o=od)
    dms = time_events(dec, args.decode_steps, 5, torch)
    Nd, Hd, D = I.DECODE_N, I.DECODE_H, I.DECODE_D
    dbytes = Nd * Hd * (2 * D * D * 4 + 6 * D * 4 + D * 4)
    dgbs = dbytes / (dms * 1e-3) / 1e9
    # the same step from a cold last-level cache: single steps, each after a
    # 512 MiB scratch write
    dcold_ms = time_cold(dec, 20, torch)
    # steady state over two states of 256 MiB each, used in turn: each step
    # reads the state the previous step did not touch, and 512 MiB of states
    # exceed the 256 MB last-level cache
    S2 = S.clone()
    states = (S, S2)

    def dec_alt():
        x = pool[it[0] % len(pool)]
        G.gdr2_decode_step(*x, states[it[0] & 1], o=od)
        it[0] += 1
    dalt_ms = time_events(dec_alt, args.decode_steps, 6, torch)
    del S2

    # the same decode step with the output epilogue fused into its store
    zd = torch.randn((Nd, Hd, D), generator=torch.Generator("cpu").manual_seed(5)).to(dev)
    nwd = torch.ones(D, dtype=torch.float32, device=dev)

    def dec_gated():
        x = pool[it[0] % len(pool)]
        it[0] += 1
        G.gdr2_decode_step_norm_gate(*x, S, zd, nwd, 1e-6, y=od)
    gms = time_events(dec_gated, args.decode_steps, 5, torch)
    gbytes = dbytes + Nd * Hd * D * 4 + D * 4
    ggbs = gbytes / (gms * 1e-3) / 1e9
    del S, pool

    # ---- output epilogue over the forward's o: RMSNorm per head + SiLU gate ----------
    _, z_epi, w_epi = I.epilogue_inputs((B, T, H, dv), seed=6)
    z_epi, w_epi = z_epi.to(dev), w_epi.to(dev)
    y_epi = torch.empty_like(o)
    fwd()
    epi = lambda: G.gdr2_norm_gate(o, z_epi, w_epi, 1e-6, dv, y=y_epi)
    ems = time_events(epi, args.steps, args.warmup, torch)
    ebytes = 3 * o.numel() * o.element_size() + dv * 4
    egbs = ebytes / (ems * 1e-3) / 1e9
    del z_epi, y_epi

    # ---- 64 packed sequences (about 262K tokens) ---------------------------------------
    varlen = varlen_leg(args, torch, G, I, dev) if args.varlen == "on" else None
    packed_long = packed_long_leg(args, torch, G, I, dev) if args.packed_long == "on" else None

    ceil = None if args.no_ceilings else ceilings(torch, dev)

    calibration_copy(args, torch, dev)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl)
        cpu["single_thread"] = cpu_single_thread(wl)

    line = {
        "metric": "GDR-2 fwd tokens/s + TFLOP/s (H16,d128,T4K); decode HBM GB/s",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, fp16/bf16 MFMA, fp32 acc",
        "data": "synthetic",
        "config": {"workload": "gdr2_chunk_fwd B4 T4096 H16 dk=dv=128, bf16 q/k/v/b/w/log_alpha, "
                               "fp32 state, S0=0, chunk 64",
                   "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv,
                   "arithmetic": "inputs and o bf16; decay sum, WY diagonal solve, every "
                                 "accumulation and the state fp32; chunk matrix T on bf16 MFMA, "
                                 "causal scores on bf16 hi/lo pairs, state-pass products on fp16 "
                                 "MFMA"},
        "fwd_tflops": tflops,
        "fwd_tflops_frac_of_bf16_peak": tflops / BF16_PEAK_TFLOPS,
        "fwd_alg_bytes": byts,
        "fwd_alg_flops": flops,
        "mfma": mfma,
        "cold_mall": None if cold_ms is None else {
            "ms_per_call": cold_ms, "tokens_per_s": tokens / (cold_ms * 1e-3),
            "hbm_frac": byts / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "method": "median of single calls, each after a 512 MiB scratch write"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": "gdr2_chunk_fwd call (intra_kernel + state_kernel), "
                               "algorithmic 1792 B per head-token"},
        "decode": {"workload": "gdr2_decode_step N256 H16 dk=dv=128 fp32 state in place",
                   "steps": args.decode_steps, "us_per_step": dms * 1e3, "alg_bytes": dbytes,
                   "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                                "traffic": load_traffic("fwd", "decode_kernel<128, 128, false>")},
                   "cold": {"us_per_step": dcold_ms * 1e3,
                            "frac": dbytes / (dcold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "method": "median of 20 single steps, each after a 512 MiB scratch write"},
                   "two_states": {"us_per_step": dalt_ms * 1e3,
                                  "frac": dbytes / (dalt_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                  "method": "back-to-back steps alternating between two 256 MiB "
                                            "states (512 MiB, beyond the 256 MB last-level cache)"},
                   "norm_gate_fused": {
                       "entry": "gdr2_decode_step_norm_gate (RMSNorm over dv + SiLU gate in the store)",
                       "us_per_step": gms * 1e3, "alg_bytes": gbytes,
                       "roofline": {"bound": "hbm", "achieved": ggbs, "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": ggbs / HBM_PEAK_GBS,
                                    "traffic": load_traffic("fwd", "decode_norm_gate_kernel<128, 128, false>")}}},
        "backward": {"workload": "gdr2_chunk_bwd B4 T4096 H16 dk=dv=128 bf16 inputs, fp32 gradients "
                                 "of q, k, v, log_alpha, b, w and S0",
                     "steps": bwd_steps, "ms_per_call": bwms, "tokens_per_s": tokens / (bwms * 1e-3),
                     "alg_bytes": bw_bytes,
                     "roofline": {"bound": "hbm", "achieved": bw_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": bw_gbs / HBM_PEAK_GBS,
                                  "traffic": load_call_traffic("fwd", "bwd_state_fwd3_kernel<128, 128>",
                                                               "bwd_")}},
        "long_sequence": long_leg(args, torch, G, I, dev) if args.long == "on" else None,
        "block": {"workload": "gdr2_chunk_fwd_block B4 T4096 H16 Hv16 dk=dv=128 from projections: "
                              "q/k L2 norm, Eq. 12 decay from bf16 W_f x, sigmoid gates (flags 7)",
                  "steps": args.steps, "ms_per_call": bms, "tokens_per_s": tokens / (bms * 1e-3),
                  "alg_bytes": byts,
                  "roofline": {"bound": "hbm", "achieved": bgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": bgbs / HBM_PEAK_GBS,
                               "traffic": load_traffic("fwd", "intra_kernel<128, 128, true, 7, 1>",
                                                       "intra_kernel<128, 128, true, 8, 2>",
                                                       "state_kernel<128, 128, 2, 4, false, 1>")}},
        "epilogue": {"workload": "gdr2_norm_gate over the forward's o [B4 T4096 H16 128] bf16, "
                                 "RMSNorm per head (group 128) x weight x silu(z), into y",
                     "steps": args.steps, "us_per_call": ems * 1e3, "alg_bytes": ebytes,
                     "roofline": {"bound": "hbm", "achieved": egbs, "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": egbs / HBM_PEAK_GBS,
                                  "traffic": load_traffic("fwd", "norm_gate_kernel<1, true>")}},
        "varlen": varlen,
        "packed_long": packed_long,
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
