#!/usr/bin/env python3
"""Throughput of one Transformer-based linear-attention head-batch, forward +
backward, on one MI355X.

A step is one la_forward (saving its state) plus one la_backward over the
same resident inputs: every row of the hot path (state reduction, apply and
normalise, the backward prologue, dQ, the gradient-state reduction, dK and
dV).  Default workload: B=4, H=16, N=4096, D=128, fp32 storage,
non-causal, i.i.d. N(0,1)/sqrt(D) inputs (dO unscaled) drawn on the GPU
from the shared seeded generator.

Output: one JSON line on stdout.  `value` is tokens/s = B*N per step / step
time over K timed steps bracketed by device synchronisation, after W untimed
warm-up steps (200 by default: the GPU reaches the clocks it holds under
sustained load only after the first few tens of steps from idle).  `roofline`
gives the dominant kernel's achieved rate from per-launch HIP events (a
second timed pass in which the library records caller-owned events around
every launch), against the MI355X fp32-MFMA or HBM peak.  `cpu_baseline`
times the fp64 CPU oracle on the host.  `variants` times the other storage
type and mask at the same shape, each after its own clock-settle phase;
`pieces` times the causal step streamed as
equal pieces through the carried-state calls (la_forward_segment /
la_backward_segment); `decode` times one recurrent decode step
(la_decode_step) per head at the bench's B x H heads and at B = 64; `layer`
times one whole layer (projections, attention, their gradients) with
C = H * D.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LA fwd+bwd tokens/s at B4 H16 D128 N4096; % of binding HBM/FLOP roofline"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix (= fp32 vector) peak
PEAK_BF16_MFMA_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
KERNEL_SOURCES = [os.path.join(ROOT, "linear_attention_transformer_amd", "csrc", f)
                  for f in ("la_kernels.hpp", "la_kernels_nc.hpp", "la_kernels_causal.hpp",
                            "la_kernels_bf16.hpp", "la_kernels_decode.hpp",
                            "la_kernels_stage.hpp", "la_api.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_MIB = 256                  # plain streaming kernel: reads and writes this much

# device kernel (demangled name) -> launch name the library's tracer reports
KERNEL_NAMES = [
    (r"k_reduce_nc<[^>]*, (true|1)>|k_reduce_bf<\d+, true>",
     "grad_state_local"),
    (r"k_reduce_nc<|k_reduce_bf<|k_state_local<", "state_local"),
    (r"k_apply_nc<[^>]*, 0>|k_apply_bf<\d+, 0>|k_fwd_causal|k_forward<", "forward"),
    (r"k_bwd_q_nc<|k_bwd_q_bf<|k_apply_bf<\d+, 1>|k_bwd_q_causal|k_bwd_q<", "bwd_q"),
    (r"k_apply_nc<[^>]*, 2>|k_apply_bf<\d+, 2>|k_bwd_kv_causal|k_bwd_kv<", "bwd_kv"),
    (r"k_state_scan", "state_scan"),
    (r"k_pad<|k_unpad<|k_stage_record", "stage"),
    (r"k_decode", "decode"),
]


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are left
    out, so that an edit of a comment keeps the traffic entries measured on
    the same code."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def algorithmic(kernel: str, BH: int, N: int, D: int, s: int, fused_bwd_q: bool):
    """(flops, bytes) per launch that the method itself requires (rows a2..a7
    of the hot path); recomputation and scans count as overhead."""
    nd, ndd = BH * N * D, BH * N * D * D
    table = {
        "state_local": (2 * ndd, 2 * nd * s),            # S = K^T V, z, u
        "forward": (2 * ndd, 2 * nd * s),                # Q S, normalise, write O
        "bwd_q": ((4 if fused_bwd_q else 2) * ndd, 3 * nd * s),  # dQ (+ dS = Q^T A)
        "grad_state_local": (2 * ndd, 2 * nd * s),       # dS when not fused
        "bwd_kv": (4 * ndd, 4 * nd * s),                 # dK, dV
        "state_scan": (0, 0),
    }
    return table.get(kernel, (0, 0))


def launch_name(kernel: str):
    import re
    for pat, name in KERNEL_NAMES:
        if re.search(pat, kernel):
            return name
    return None


def workload_key(kernel, B, H, N, D, dtype, causal):
    return "%s B%d H%d N%d D%d %s causal=%d" % (kernel, B, H, N, D, dtype, int(causal))


def pmc_summary(fetch_dir, write_dir, args):
    """Per-launch HBM traffic of the library's kernels from two rocprofv3
    --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch).  Each counter is scaled by what it reads for the copy kernel
    the same run launches (COPY_MIB read and COPY_MIB written), so the
    figures are bytes.  Merges the entries into profiles/traffic.json and
    prints a markdown table."""
    import csv
    import glob

    def load(d, counter):
        per, calib = {}, []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                val = float(r["Counter_Value"])
                if "neg_kernel" in r["Kernel_Name"]:
                    calib.append(val)
                name = launch_name(r["Kernel_Name"]) if "la::" in r["Kernel_Name"] else None
                if name:
                    per.setdefault(name, []).append(val)
        if not calib:
            sys.exit("bench.py: no copy-kernel dispatch with %s under %s" % (counter, d))
        return {n: sum(v) / len(v) for n, v in per.items()}, sum(calib) / len(calib), \
            {n: len(v) for n, v in per.items()}

    fetch, fcal, count = load(fetch_dir, "FETCH_SIZE")
    write, wcal, _ = load(write_dir, "WRITE_SIZE")
    copy_bytes = COPY_MIB << 20
    fs, wsc = copy_bytes / (fcal * 1024), copy_bytes / (wcal * 1024)
    doc = {"entries": {}}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            doc = json.load(f)
    if doc.get("kernel_source_hash") != kernel_source_hash():
        doc = {"entries": {}}
    doc["kernel_source_hash"] = kernel_source_hash()
    doc["calibration"] = {"copy_bytes_each_way": copy_bytes, "fetch_kib": fcal,
                          "write_kib": wcal, "fetch_scale": fs, "write_scale": wsc}
    s = 4 if args.dtype == "fp32" else 2
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | write MB "
          "| traffic MB | algorithmic MB |")
    print("|---|---|---|---|---|---|---|---|")
    for name in sorted(fetch):
        rd, wr = fetch[name] * 1024 * fs, write.get(name, 0.0) * 1024 * wsc
        key = workload_key(name, args.B, args.H, args.N, args.D, args.dtype, args.causal)
        doc["entries"][key] = {"bytes_per_launch": round(rd + wr), "read_bytes": round(rd),
                               "write_bytes": round(wr)}
        alg = algorithmic(name, args.B * args.H, args.N, args.D, s,
                          "grad_state_local" not in fetch)[1]
        print("| %s | %d | %.0f | %.0f | %.1f | %.1f | %.1f | %.1f |"
              % (name, count[name], fetch[name], write.get(name, 0.0), rd / 1e6, wr / 1e6,
                 (rd + wr) / 1e6, alg / 1e6))
    print("\ncalibration: copy kernel of %d MiB each way read FETCH_SIZE %.0f KiB, "
          "WRITE_SIZE %.0f KiB -> scales %.3f, %.3f" % (COPY_MIB, fcal, wcal, fs, wsc))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(doc, f, indent=1, sort_keys=True)


COUNTERS = ("SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F32 "
            "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
            "GRBM_GUI_ACTIVE")


def counter_summary(pmc_dir, args):
    """Per-launch matrix-core and instruction counts of the library's kernels
    from one rocprofv3 --pmc run of this script with COUNTERS (no GPU work).
    MOPS count MFMA work in units of 512 flops; the MFMA busy fraction is
    SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE (summed over the 8 XCDs)
    times the 1024 SIMDs."""
    import collections
    import csv
    import glob
    import statistics as st
    f = glob.glob(os.path.join(pmc_dir, "*counter_collection.csv"))[0]
    by = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(f)):
        n = r["Kernel_Name"]
        if "la::" not in n:
            continue
        name = launch_name(n.split("(")[0].replace("void ", ""))
        by[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[name][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    s = 4 if args.dtype == "fp32" else 2
    B, H, N, D = args.B, args.H, args.N, args.D
    fused = "grad_state_local" not in by
    print("| kernel | us | MFMA instr | MOPS x 512 / algorithmic flops | MFMA busy | "
          "VALU (non-MFMA) / MFMA | LDS / MFMA | SALU / MFMA | TFLOP/s |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, c in by.items():
        m = {k: st.mean(v) for k, v in c.items()}
        t = st.mean(dur[name].values()) * 1e-9
        mops = m.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0) + m.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0)
        flops, _ = algorithmic(name, B * H, N, D, s, fused)
        mf = m.get("SQ_INSTS_MFMA", 0)
        g = m.get("GRBM_GUI_ACTIVE", 0) / 8
        per = lambda k: (m.get(k, 0) / mf) if mf else float("nan")  # noqa: E731
        print("| %s | %.1f | %.3g | %s | %s | %.2f | %.2f | %.2f | %s |" % (
            name, t * 1e6, mf, "%.3f" % (mops * 512 / flops) if flops else "-",
            "%.3f" % (m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / (g * 1024)) if g else "-",
            (m.get("SQ_INSTS_VALU", 0) - mf) / mf if mf else float("nan"),
            per("SQ_INSTS_LDS"), per("SQ_INSTS_SALU"),
            "%.1f" % (mops * 512 / t / 1e12) if t else "-"))


LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS "
                "SQ_WAIT_INST_LDS SQ_LDS_MEM_VIOLATIONS SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE")


def lds_summary(pmc_dir, args):
    """Per-launch LDS counters of the library's kernels from one rocprofv3
    --pmc run of this script with LDS_COUNTERS (no GPU work): bank-conflict
    stall cycles over the cycles the LDS did useful indexed work
    (SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT)), the
    LDS busy fraction (SQ_LDS_IDX_ACTIVE over GRBM_GUI_ACTIVE / 8 cycles of
    one XCD times 256 compute units), address-conflict cycles, issue-wait
    cycles per LDS instruction (SQ_WAIT_INST_LDS counts 4-cycle units) and
    the LDS memory violations (0 when every access is in range)."""
    import collections
    import csv
    import glob
    import statistics as st
    f = glob.glob(os.path.join(pmc_dir, "*counter_collection.csv"))[0]
    by = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in csv.DictReader(open(f)):
        n = r["Kernel_Name"]
        if "la::" not in n:
            continue
        name = launch_name(n.split("(")[0].replace("void ", ""))
        by[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[name][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    print("| kernel | us | LDS instr | bank-conflict / useful LDS cycles | LDS busy | "
          "address-conflict cycles | wait cycles per LDS instr | LDS violations |")
    print("|---|---|---|---|---|---|---|---|")
    for name, c in by.items():
        m = {k: st.mean(v) for k, v in c.items()}
        t = st.mean(dur[name].values()) * 1e-9
        bank, idx = m.get("SQ_LDS_BANK_CONFLICT", 0), m.get("SQ_LDS_IDX_ACTIVE", 0)
        g = m.get("GRBM_GUI_ACTIVE", 0) / 8
        ni = m.get("SQ_INSTS_LDS", 0)
        print("| %s | %.1f | %.3g | %s | %s | %.3g | %s | %d |" % (
            name, t * 1e6, ni, "%.3f" % (bank / (idx - bank)) if idx > bank else "-",
            "%.3f" % (idx / (g * 256)) if g else "-", m.get("SQ_LDS_ADDR_CONFLICT", 0),
            "%.2f" % (4 * m.get("SQ_WAIT_INST_LDS", 0) / ni) if ni else "-",
            int(sum(c.get("SQ_LDS_MEM_VIOLATIONS", [0])))))


def copy_reference(dev):
    """Bandwidth of a plain streaming kernel (torch.neg over COPY_MIB fp32,
    read once and written once): the achievable-HBM reference, and the
    calibration dispatch for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = (COPY_MIB << 20) // 4
    src = torch.zeros(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    reps = 5
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps * 1e-3
    del src, dst
    return 2 * (COPY_MIB << 20) / t / 1e9


def uses_bf16_mfma(dtype, D, causal):
    """Whether every kernel of the path computes on the bf16 matrix cores
    (bf16 storage, 32 <= D <= 128, either mask); otherwise fp32 matrix cores."""
    return dtype == "bf16" and 32 <= D <= 128


def step_floor_us(B, H, N, D, s, bf16_mfma):
    """Roofline time of one fwd+bwd step: algorithmic bytes at the HBM peak
    against algorithmic flops at the matrix peak of the operand type."""
    flops, nbytes = 12 * B * H * N * D * D, 11 * B * H * N * D * s
    peak = PEAK_BF16_MFMA_TFLOPS if bf16_mfma else PEAK_FP32_MFMA_TFLOPS
    return 1e6 * max(flops / (peak * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))


FLUSH_MIB = 512                 # scratch written between flushed steps (> 256 MB MALL)


def measure(fn, steps, warmup, flush=None):
    """Time `steps` calls of fn.  Unflushed: the calls back to back between
    two device synchronisations, with an event before each call and after
    the last, so one region gives the mean (total / steps) and the median of
    the per-call times.  Flushed (when `flush`, a device buffer, is given):
    each call preceded by a write of the whole buffer, which evicts the
    inputs from the L2 caches and the MALL, and timed between its own two
    events.  Returns a dict of ms."""
    import statistics
    import torch
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    out = {"mean": ev[0].elapsed_time(ev[-1]) / steps, "median": statistics.median(per)}
    if flush is not None:
        a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            flush.fill_(float(i & 7))
            a[i].record()
            fn()
            b[i].record()
        torch.cuda.synchronize()
        per = [a[i].elapsed_time(b[i]) for i in range(steps)]
        out["flushed_mean"] = sum(per) / steps
        out["flushed_median"] = statistics.median(per)
    return out


def pass_floor_us(kind, B, H, N, D, s, bf16_mfma):
    """Roofline time of the forward (4ND^2 flops, 4ND*s bytes per head) or
    the backward (8ND^2, 7ND*s) alone."""
    f, b = {"forward": (4, 4), "backward": (8, 7)}[kind]
    flops, nbytes = f * B * H * N * D * D, b * B * H * N * D * s
    peak = PEAK_BF16_MFMA_TFLOPS if bf16_mfma else PEAK_FP32_MFMA_TFLOPS
    return 1e6 * max(flops / (peak * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))


def fp16_step_floor_us(B, H, N, D):
    """Roofline time of the fp16-storage step at 32 <= D <= 128 non-causal,
    priced on the arithmetic it runs: the two segment reductions (S and dS,
    2ND^2 each) on the fp32 matrix cores; the forward apply, the dQ role and
    dK | dV (8ND^2 in all) as split products, six bf16 matrix products per
    fp32 product; against 11ND*2 bytes at the HBM peak."""
    nd2 = B * H * N * D * D
    t_mfma = 4 * nd2 / (PEAK_FP32_MFMA_TFLOPS * 1e12) + 6 * 8 * nd2 / (PEAK_BF16_MFMA_TFLOPS * 1e12)
    return 1e6 * max(t_mfma, 11 * B * H * N * D * 2 / (PEAK_HBM_GBS * 1e9))


def settle(step, seconds):
    """Clock settle: untimed calls of step for a fixed wall time (synchronised
    every 16 calls, so the host does not run far ahead).  Returns the count."""
    import torch
    n = 0
    t_end = time.perf_counter() + max(seconds, 0.0)
    while time.perf_counter() < t_end:
        step()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_variant(la, make_inputs, dev, B, H, N, D, dtype, causal, steps, warmup, settle_s):
    """ms per fwd+bwd step of another storage type / mask at the same shape
    (same protocol as the headline: clock settle, warm-up, then the steps back
    to back)."""
    import torch
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=0, device=dev, draw_device=dev)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    ws = la.alloc_workspace(B, H, N, D, causal, dev, dtype)
    st = torch.empty(max(la.state_size(B, H, N, D, causal) // 4, 4), dtype=torch.float32,
                     device=dev)

    def step():
        la.forward(q, k, v, causal, out=o, state_out=st, workspace=ws)
        la.backward(q, k, v, g, causal, state=st, outs=(dq, dk, dv), workspace=ws)

    n = settle(step, settle_s)
    r = measure(step, steps, warmup)
    r["settle_steps"] = n
    return r


def time_pieces(la, make_inputs, dev, B, H, N, D, dtype, pieces, steps, warmup):
    """ms per causal fwd+bwd step of the same workload streamed as `pieces`
    equal pieces through the carried-state calls: forward in order, each piece
    taking the previous one's record; backward in reverse, each taking the
    next piece's gradient record.  Inputs are split into per-piece tensors
    before timing."""
    import torch
    q, k, v, g = make_inputs(B, H, N, D, dtype=dtype, seed=0, device=dev, draw_device=dev)
    n = N // pieces
    sl = [slice(i * n, N if i == pieces - 1 else (i + 1) * n) for i in range(pieces)]
    parts = [[x[:, :, c].contiguous() for x in (q, k, v, g)] for c in sl]
    del q, k, v, g
    outs = [[torch.empty_like(p[0]) for _ in range(4)] for p in parts]
    recs = [la.new_record(B, H, D, dev) for _ in range(pieces)]
    grecs = [la.new_record(B, H, D, dev) for _ in range(pieces)]
    ws = max((la.alloc_workspace(B, H, c.stop - c.start, D, True, dev, dtype) for c in sl),
             key=lambda t: t.numel())
    sts = [torch.empty(max(la.state_size(B, H, c.stop - c.start, D, True) // 4, 4),
                       dtype=torch.float32, device=dev) for c in sl]

    def step():
        for i, (p, c) in enumerate(zip(parts, sl)):
            la.forward_segment(p[0], p[1], p[2], True, carry_in=recs[i - 1] if i else None,
                               n_carry=c.start, carry_out=recs[i], out=outs[i][0],
                               state_out=sts[i], workspace=ws)
        for i in reversed(range(pieces)):
            p, c = parts[i], sl[i]
            la.backward_segment(p[0], p[1], p[2], p[3], True, n_carry=c.start,
                                gcarry_in=grecs[i + 1] if i + 1 < pieces else None,
                                gcarry_out=grecs[i], state=sts[i], outs=outs[i][1:],
                                workspace=ws)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_decode(la, make_inputs, dev, B, H, D, dtype, steps, warmup):
    """One recurrent decode step (la_decode_step) per head of B x H heads,
    the state alternating between two records.  Returns (us per step issued
    from Python, us per step replayed from a captured HIP graph of 100 steps,
    HBM bytes per step).  The graph removes the host's per-call cost, so its
    time is the device's.  The algorithmic bytes are the record read and
    written once per head plus the token's q, k, v in and o out."""
    import torch
    q, k, v, _ = make_inputs(B, H, 1, D, dtype=dtype, seed=0, device=dev)
    q, k, v = (x[:, :, 0].contiguous() for x in (q, k, v))
    o = torch.empty_like(q)
    recs = [la.new_record(B, H, D, dev).zero_(), la.new_record(B, H, D, dev)]

    def run(n):
        for i in range(n):
            la.decode_step(q, k, v, recs[i % 2], state_out=recs[(i + 1) % 2], n_prev=i,
                           out=o)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run(warmup)
    eager_us = 1e3 * timed(lambda: run(steps), 1) / steps
    per_graph = 100
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run(per_graph)                      # warm the side stream
    torch.cuda.current_stream(dev).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(per_graph)
    reps = max(steps // per_graph, 1)
    graph.replay()
    graph_us = 1e3 * timed(graph.replay, reps) / (reps * per_graph)
    nbytes = 2 * B * H * (D * D + 2 * D) * 4 + 4 * B * H * D * q.element_size()
    return eager_us, graph_us, nbytes


def time_layer(la, dev, B, N, H, D, dtype, causal, steps, warmup):
    """ms per forward + backward of one linear-attention layer with C = H*D
    (la_layer_forward / la_layer_backward: QKV projection, attention, output
    projection and their gradients), and its flops per step: the six
    projection GEMMs (2*B*N*C*(3HD + HD) forward, twice that backward) plus
    the attention's 12*B*H*N*D^2."""
    import torch
    from linear_attention_transformer_amd.inputs import make_layer_inputs
    C = H * D
    x, wqkv, wo, dy = make_layer_inputs(B, N, C, H, D, dtype=dtype, seed=0, device=dev)
    sb, wb = la.layer_sizes(B, N, C, H, D, causal, dtype)
    saved = torch.empty(sb, dtype=torch.uint8, device=dev)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    outs = (torch.empty_like(x), torch.empty_like(wqkv), torch.empty_like(wo))

    def step():
        la.layer_forward(x, wqkv, wo, H, causal, saved=saved, out=y, workspace=ws)
        la.layer_backward(x, wqkv, wo, dy, H, causal, saved=saved, outs=outs, workspace=ws)

    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 3 * 2 * B * N * C * 4 * H * D + 12 * B * H * N * D * D
    return ms, flops


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(q, k, v, g, causal):
    import oracle
    from linear_attention_transformer_amd.inputs import as_f64_numpy
    B, H, N, D = q.shape
    BH = B * H
    # about 5-15 s of oracle work on a 16-core host: the whole workload at the
    # default size, proportionally fewer heads for larger N * D^2
    heads = max(1, min(BH, round(BH * (4096 * 128 * 128) / (N * D * D))))
    sel = lambda t: t.reshape(BH, N, D)[:heads].unsqueeze(0)
    a = [as_f64_numpy(sel(x)) for x in (q, k, v, g)]
    oracle.build(force=False)
    times = []
    # at least 3 runs and about 10 s of oracle work, at most 15 runs
    while len(times) < 3 or (sum(times) < 10.0 and len(times) < 15):
        t0 = time.perf_counter()
        oracle.forward_state(a[0], a[1], a[2], causal)
        oracle.backward_state(*a, causal)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    tokens = B * N * heads / BH
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "fp64 C oracle (state form, OpenMP over heads), forward+backward "
                      "of %d of the %d heads at N=%d D=%d; median of %d runs, %.2f s "
                      "each; value scaled to the workload's B*N tokens"
                      % (heads, BH, N, D, len(times), dt)}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU raises its clocks over the first tens of steps after idle
    # (measured: ~0.8 ms/step over the first 20 fp32 steps, ~0.50 ms/step
    # from about step 60 on), so the untimed warm-up is long by default
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="before the warm-up steps (of the headline and of each variant), "
                         "run steps untimed for this long so the GPU reaches its loaded "
                         "clocks (reported as clock_settle)")
    ap.add_argument("--dtype", choices=("fp32", "bf16", "fp16"), default="fp32",
                    help="storage dtype of Q, K, V, O and gradients (arithmetic is fp32; "
                         "fp16 storage is staged through fp32 buffers)")
    ap.add_argument("--causal", type=int, choices=(0, 1), default=0)
    ap.add_argument("--B", type=int, default=4)
    ap.add_argument("--H", type=int, default=16)
    ap.add_argument("--N", type=int, default=4096)
    ap.add_argument("--D", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the other storage type / mask at the same shape")
    ap.add_argument("--pieces", type=int, default=4,
                    help="also time the causal step of this shape and storage streamed as "
                         "this many pieces through the carried-state calls (0 = skip)")
    ap.add_argument("--counter-summary", metavar="PMC_DIR",
                    help="summarise one rocprofv3 --pmc run of this script with the counters "
                         "of COUNTERS (matrix-core work and busy cycles, VALU, LDS and SALU "
                         "instructions per kernel) as a markdown table; no GPU work")
    ap.add_argument("--lds-summary", metavar="PMC_DIR",
                    help="summarise one rocprofv3 --pmc run of this script with the counters "
                         "of LDS_COUNTERS (bank and address conflicts, LDS busy, issue waits) "
                         "as a markdown table; no GPU work")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of this script (FETCH_SIZE, "
                         "WRITE_SIZE) for the given workload into profiles/traffic.json; "
                         "no GPU work")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args)
        return
    if args.lds_summary:
        lds_summary(args.lds_summary, args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library measures the linear-attention hot path on one GPU "
              "(heads shard across GPUs with no communication); --gpus %d is not "
              "supported" % max(args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_attention_transformer_amd as la
    from linear_attention_transformer_amd.inputs import make_inputs
    if not os.path.exists(la.LIB_PATH):
        from linear_attention_transformer_amd import build as hip_build
        hip_build.build()
    la.load_library()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, N, D, causal = args.B, args.H, args.N, args.D, bool(args.causal)
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[args.dtype]
    s = 4 if args.dtype == "fp32" else 2
    print("bench: B=%d H=%d N=%d D=%d %s causal=%d steps=%d warmup=%d"
          % (B, H, N, D, args.dtype, causal, args.steps, args.warmup), file=sys.stderr, flush=True)
    q, k, v, g = make_inputs(B, H, N, D, dtype=dt, seed=0, device=dev, draw_device=dev)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    ws = la.alloc_workspace(B, H, N, D, causal, dev, dt)
    st = torch.empty(max(la.state_size(B, H, N, D, causal) // 4, 4), dtype=torch.float32,
                     device=dev)

    def step(tf=None, tb=None):
        la.forward(q, k, v, causal, out=o, state_out=st, workspace=ws, trace=tf)
        la.backward(q, k, v, g, causal, state=st, outs=(dq, dk, dv), workspace=ws, trace=tb)

    # clock settle (untimed steps for a fixed wall time), then the warm-up steps
    settle_steps = settle(step, args.settle_s)
    # device memory of the step: the 8 I/O tensors plus the library's
    # workspace and saved state (everything the caller allocates for it)
    mem = {"peak_allocated": torch.cuda.max_memory_allocated(dev),
           "io_tensors": 8 * q.numel() * q.element_size(),
           "workspace": ws.numel(), "saved_state": st.numel() * 4}

    # timed region 1: the headline, nothing but the K steps (after the W
    # warm-up steps), back to back between two synchronisations
    w0 = time.perf_counter()
    head = measure(step, args.steps, args.warmup)
    wall = time.perf_counter() - w0
    ms = head["mean"]
    tokens_per_s = B * N / (ms * 1e-3)
    print("bench: %.3f ms/step (median %.3f; wall incl. warm-up %.3f ms/step), %.1f M tokens/s"
          % (ms, head["median"], wall * 1e3 / (args.steps + args.warmup), tokens_per_s / 1e6),
          file=sys.stderr, flush=True)
    # the same steps with the L2 caches and the MALL flushed before each
    flush = torch.empty((FLUSH_MIB << 20) // 4, dtype=torch.float32, device=dev)
    fl = measure(step, args.steps, 0, flush=flush)
    print("bench: flushed %.3f ms/step (median %.3f)" % (fl["flushed_mean"], fl["flushed_median"]),
          file=sys.stderr, flush=True)

    # timed region 2: the same K steps with per-launch events
    traces = [(la.KernelTrace(dev), la.KernelTrace(dev)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for tf, tb in traces:
        step(tf, tb)
    t1.record()
    torch.cuda.synchronize()
    traced_ms = t0.elapsed_time(t1) / args.steps
    per_kernel = {}
    for tf, tb in traces:
        for tr in (tf, tb):
            for name, t in zip(tr.names(), tr.times_ms()):
                per_kernel.setdefault(name, []).append(t)
    launches = {n: len(v) // args.steps for n, v in per_kernel.items()}
    avg_us = {n: 1e3 * sum(v) / len(v) for n, v in per_kernel.items()}
    step_us = {n: avg_us[n] * launches[n] for n in avg_us}
    dom = max(step_us, key=step_us.get)
    fused = "grad_state_local" not in per_kernel   # dQ kernel also reduces dS
    flops, nbytes = algorithmic(dom, B * H, N, D, s, fused)
    t_dom = avg_us[dom] * 1e-6
    bf16_mfma = uses_bf16_mfma(args.dtype, D, causal)
    mpeak = PEAK_BF16_MFMA_TFLOPS if bf16_mfma else PEAK_FP32_MFMA_TFLOPS
    ridge = mpeak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if nbytes and flops / nbytes < ridge:
        bound, achieved, peak, unit = "hbm", nbytes / t_dom / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", flops / t_dom / 1e12, mpeak, "TFLOP/s"
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        key = workload_key(dom, B, H, N, D, args.dtype, causal)
        ent = tr.get("entries", {}).get(key)
        if ent and tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = ent["bytes_per_launch"]
    roofline = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom,
                "kernel_avg_us": round(avg_us[dom], 2),
                "algorithmic_per_launch": {"flops": flops, "bytes": nbytes}}
    floor_us = step_floor_us(B, H, N, D, s, bf16_mfma)
    if args.dtype == "fp16" and 32 <= D <= 128 and not causal:
        floor_us = fp16_step_floor_us(B, H, N, D)
    # the step's own fraction beside the dominant kernel's
    roofline["step"] = {"floor_us": round(floor_us, 1), "frac": round(floor_us / (ms * 1e3), 4)}
    print("bench: per-kernel us/launch " + ", ".join("%s=%.1f" % kv for kv in avg_us.items()),
          file=sys.stderr, flush=True)

    # the forward and the backward alone, both masks, same storage; each
    # against its own floor, unflushed and flushed
    passes = {}
    if not args.no_variants:
        for pc in (False, True):
            pws = la.alloc_workspace(B, H, N, D, pc, dev, dt)
            pst = torch.empty(max(la.state_size(B, H, N, D, pc) // 4, 4), dtype=torch.float32,
                              device=dev)
            la.forward(q, k, v, pc, out=o, state_out=pst, workspace=pws)
            fns = {"forward": lambda: la.forward(q, k, v, pc, out=o, state_out=pst,
                                                 workspace=pws),
                   "backward": lambda: la.backward(q, k, v, g, pc, state=pst,
                                                   outs=(dq, dk, dv), workspace=pws)}
            for kind, fn in fns.items():
                r = measure(fn, args.steps, args.warmup, flush=flush)
                pf = pass_floor_us(kind, B, H, N, D, s, bf16_mfma)
                passes["%s %s" % (kind, "causal" if pc else "non-causal")] = {
                    "ms": round(r["mean"], 4), "ms_median": round(r["median"], 4),
                    "ms_flushed_median": round(r["flushed_median"], 4),
                    "tokens_per_s": round(B * N / (r["mean"] * 1e-3), 1),
                    "floor_us": round(pf, 1), "frac": round(pf / (r["mean"] * 1e3), 4)}
                print("bench: %s %s alone: %.3f ms (flushed %.3f), %.2f of its floor"
                      % (kind, "causal" if pc else "non-causal", r["mean"], r["flushed_median"],
                         pf / (r["mean"] * 1e3)), file=sys.stderr, flush=True)
            del pws, pst

    # the other storage type and mask at the same shape, each timed like the
    # headline (bf16 storage runs on the bf16 matrix cores for 32 <= D <= 128)
    variants = {}
    if not args.no_variants:
        del o, dq, dk, dv, ws, st
        torch.cuda.empty_cache()
        combos = [(vdt, vc) for vdt in ("fp32", "bf16") for vc in (False, True)]
        combos.append(("fp16", False))
        for vdt, vc in combos:
            if vdt == args.dtype and vc == causal:
                continue
            tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[vdt]
            r = time_variant(la, make_inputs, dev, B, H, N, D, tdt, vc, args.steps,
                             args.warmup, args.settle_s)
            vms = r["mean"]
            vs = 4 if vdt == "fp32" else 2
            if vdt == "fp16" and 32 <= D <= 128 and not vc:
                vfl, basis = fp16_step_floor_us(B, H, N, D), "fp32 + split-bf16 matrix cores"
            else:
                bm = uses_bf16_mfma(vdt, D, vc)
                vfl = step_floor_us(B, H, N, D, vs, bm)
                basis = "bf16 matrix cores / HBM" if bm else "fp32 matrix cores / HBM"
            variants["%s %s" % (vdt, "causal" if vc else "non-causal")] = {
                "ms_per_step": round(vms, 4), "ms_median": round(r["median"], 4),
                "tokens_per_s": round(B * N / (vms * 1e-3), 1),
                "step_floor_us": round(vfl, 1), "step_frac": round(vfl / (vms * 1e3), 4),
                "floor_basis": basis,
                "clock_settle": {"seconds": args.settle_s, "steps": r["settle_steps"]}}
            print("bench: variant %s %s: %.3f ms/step" % (vdt, "causal" if vc else
                  "non-causal", vms), file=sys.stderr, flush=True)

    # the causal step streamed in pieces through the carried-state calls,
    # against the same step over the whole sequence
    pieces = None
    if not args.no_variants and args.pieces > 1:
        torch.cuda.empty_cache()
        pms = time_pieces(la, make_inputs, dev, B, H, N, D, dt, args.pieces,
                          max(args.steps // 2, 5), args.warmup)
        whole = ms if causal else variants.get("%s causal" % args.dtype, {}).get("ms_per_step")
        pieces = {"pieces": args.pieces, "causal": True, "ms_per_step": round(pms, 4),
                  "whole_sequence_ms_per_step": None if whole is None else round(whole, 4),
                  "tokens_per_s": round(B * N / (pms * 1e-3), 1),
                  "vs_whole": None if whole is None else round(whole / pms, 4)}
        print("bench: causal %s in %d pieces: %.3f ms/step (whole sequence %s)"
              % (args.dtype, args.pieces, pms, whole), file=sys.stderr, flush=True)

    # one whole layer around the attention (projections on rocBLAS)
    layer = None
    if not args.no_variants:
        torch.cuda.empty_cache()
        lms, lfl = time_layer(la, dev, B, N, H, D, dt, causal, max(args.steps // 4, 5),
                              max(args.warmup // 10, 5))
        lpeak = PEAK_FP32_MFMA_TFLOPS if args.dtype == "fp32" else PEAK_BF16_MFMA_TFLOPS
        gemm_fl = lfl - 12 * B * H * N * D * D
        layer = {"C": H * D, "ms_per_step": round(lms, 4),
                 "tokens_per_s": round(B * N / (lms * 1e-3), 1),
                 "flops_per_step": lfl, "achieved_TFLOPs": round(lfl / (lms * 1e-3) / 1e12, 1),
                 "peak_TFLOPs": lpeak, "frac": round(lfl / (lms * 1e-3) / 1e12 / lpeak, 4),
                 "attention_ms_per_step": round(ms, 4),
                 # the step split: the attention timed alone on the same
                 # shapes, the projections' GEMMs the rest; no pass moves rows
                 # between layouts
                 "breakdown_ms": {"attention": round(ms, 4), "gemms": round(lms - ms, 4),
                                  "layout_passes": 0.0},
                 "gemm_TFLOPs": round(gemm_fl / ((lms - ms) * 1e-3) / 1e12, 1)
                 if lms > ms else None}
        print("bench: layer (C=%d) fwd+bwd %.3f ms/step, %.0f TFLOP/s (attention alone %.3f ms)"
              % (H * D, lms, lfl / (lms * 1e-3) / 1e12, ms), file=sys.stderr, flush=True)

    # the recurrent decode step at the bench's heads and at a serving batch
    decode = None
    if not args.no_variants:
        decode = {}
        for db in (B, 64):
            eus, us, nb = time_decode(la, make_inputs, dev, db, H, D, dt, 2000, args.warmup)
            decode["B%d H%d" % (db, H)] = {
                "us_per_step": round(us, 2), "us_per_step_eager": round(eus, 2),
                "tokens_per_s": round(db / (us * 1e-6), 1),
                "hbm_bytes_per_step": nb, "achieved_GBs": round(nb / (us * 1e-6) / 1e9, 1),
                "frac_of_hbm_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            print("bench: decode step B=%d H=%d D=%d %s: %.2f us in a graph (%.0f GB/s), "
                  "%.2f us issued one by one" % (db, H, D, args.dtype, us,
                                                 nb / (us * 1e-6) / 1e9, eus),
                  file=sys.stderr, flush=True)

    # the copy reference runs after every timed region: a burst of streaming
    # traffic just before one would lower its clocks
    copy_gbs = copy_reference(dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, k, v, g, causal)
        print("bench: cpu baseline %.3g tokens/s on %d threads" % (cpu["value"], cpu["cores"]),
              file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16_mfma else "f32",
        "data": "synthetic",
        "config": {"workload": "LA forward+backward, B=%d H=%d N=%d D=%d, %s storage, %s"
                               % (B, H, N, D, args.dtype, "causal" if causal else "non-causal"),
                   "B": B, "H": H, "N": N, "D": D, "causal": causal, "storage": args.dtype,
                   "global_batch": B, "seq_len": N},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "step_roofline": {"floor_us": round(floor_us, 1),
                          "frac": round(floor_us / (ms * 1e3), 4)},
        "ms_per_step_median": round(head["median"], 4),
        "flushed": {"ms_per_step": round(fl["flushed_mean"], 4),
                    "ms_per_step_median": round(fl["flushed_median"], 4),
                    "scratch_written_MiB": FLUSH_MIB},
        "clock_settle": {"seconds": args.settle_s, "steps": settle_steps},
        "passes": passes,
        "kernels_us_per_launch": {n: round(t, 2) for n, t in avg_us.items()},
        "traced_ms_per_step": round(traced_ms, 4),
        "hbm_copy_GBs": round(copy_gbs, 1),
        "memory_bytes": mem,
        "variants": variants,
        "pieces": pieces,
        "decode": decode,
        "layer": layer,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
