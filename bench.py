#!/usr/bin/env python3
"""Benchmark of the chunked gated-delta-rule forward pass on one MI355X.

One step = one call of gdn_chunk_fwd (kda_chunk_fwd for the KDA workload) over
the whole synthetic batch: the prepare kernel and the fused state/output
kernel, inputs resident in HBM, workspace preallocated. Prints one JSON line.

Timing: each of the K timed calls is bracketed by its own HIP events on the
call's stream, with a 1 GiB buffer read before it, so that the inputs come
from HBM rather than the 256 MB last-level cache and the caches hold only
clean lines; the headline is the median (p10 and p90 reported beside it). A
second scrubbed pass of K calls, with the library recording HIP events around
each kernel on the launch stream, gives the per-kernel durations (kept out of
the headline pass, whose calls they would lengthen). Two more passes are
reported beside the headline: the K calls with the 1 GiB buffer written
instead of read before each (the caches then hold dirty lines of other data,
whose write-back the call pays for), and the K calls back to back with no
scrub ("warm"). The host side of a call (argument checks, the packed
input's chunk table build and upload, the launches) is timed on its own with
the GPU drained before each call ("host_call_us").

    python bench.py [--steps K] [--warmup W] [--workload gdn|varlen|long|kda|tiny]
                    [--no-cpu-baseline]

The default workload is B=4 T=4096 H=16 K=V=128 (GDN, in-kernel L2-norm and
sigmoid(beta), final state on), the configuration the headline metric is
quoted on. Only one GPU is used: --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd tokens/s, GDN H=16 K=V=128 T=4096 B=4; % bf16 MFMA peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix

# Algorithmic work per token-head (q, k, v bf16 + gate + beta + o bf16), and
# its split between the two kernels by first touch of the algorithm's inputs
# and outputs: prepare reads q, k, g, beta; the state/output kernel reads v
# and writes o and the states.
GDN_PREP_BYTES = 256 + 256 + 4 + 2
KDA_PREP_BYTES = 256 + 256 + 512 + 2
STATE_BYTES = 256 + 256
STATE_BYTES_PER_UNIT = 128 * 128 * 4  # one fp32 state per (sequence, head), each of initial/final
ALG_FLOPS_PER_TH = 140629             # conservative (triangle-exploiting) count


FWD_SOURCES = ("gdn_common.h", "gdn_kernels.h", "gdn_prepare.hip", "gdn_fwd.hip", "gdn_state.hip",
               "gdn_state_common.h", "kda_fwd.hip", "kda_state.hip")
KERNEL_SOURCES = FWD_SOURCES + ("gdn_bwd.h", "gdn_bwd.hip", "short_conv.hip", "kda_bwd.hip")


def sources_for(workload: str):
    """The kernel sources a workload's counter summary depends on."""
    if workload == "bwd_kda":
        return FWD_SOURCES + ("gdn_bwd.h", "gdn_bwd.hip", "kda_bwd.hip")
    if workload.startswith("bwd"):
        return FWD_SOURCES + ("gdn_bwd.h", "gdn_bwd.hip")
    if workload == "conv":
        return ("gdn_common.h", "gdn_kernels.h", "short_conv.hip")
    return FWD_SOURCES


def kernel_source_hash(workload=None) -> str:
    """Hash of the kernel sources (of one workload's kernels, or all); HBM
    counters recorded for other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES if workload is None else sources_for(workload)):
        with open(os.path.join(ROOT, "chunked_gated_delta_03_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, kernel_name_part: str):
    """Scaled HBM bytes per launch of a kernel from the committed counter
    summary of this workload, or None if absent or taken on other sources."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.json")):
        with open(path) as f:
            d = json.load(f)
        if d.get("workload") != workload or d.get("kernel_source_hash") != kernel_source_hash(workload):
            continue
        for name, rec in d["kernels"].items():
            if kernel_name_part in name:
                return rec["hbm_bytes_scaled"]
    return None


def recorded_mfma(workload: str, kernel_name_part: str):
    """MFMA counters of a kernel from the committed summary of this workload
    (``profiles/*_mfma_counters.json``): the fraction of the SIMDs' cycles
    their matrix units were busy during the kernel, or None if absent or
    taken on other sources."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_mfma_counters.json")):
        with open(path) as f:
            d = json.load(f)
        if d.get("workload") != workload or d.get("kernel_source_hash") != kernel_source_hash(workload):
            continue
        for name, rec in d["kernels"].items():
            if kernel_name_part in name:
                return rec["mfma_busy_frac"]
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gdn", choices=["gdn", "varlen", "long", "kda", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--op", default="fwd", choices=["fwd", "summary", "conv", "bwd"],
                    help="fwd: the forward pass (default); summary: the affine state summary and its apply step; "
                         "conv: the causal depthwise Conv1d + SiLU forming q, k, v (D = 3*H*128, W = 4); "
                         "bwd: the GDN backward pass")
    ap.add_argument("--gate-in-kernel", action="store_true",
                    help="fwd: call the gated entry (raw gate, A_log, dt_bias; the gate formed in the kernel)")
    ap.add_argument("--scrub-mib", type=int, default=1024, help="MiB read between timed calls (0: none)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run plain device-to-device copies of this many MiB (counter calibration)")
    return ap.parse_args()


def calibrate_copy(mib: int, reps: int = 5) -> None:
    """Plain copies of a known size: the FETCH_SIZE / WRITE_SIZE counters of
    this copy kernel give the scale factor between counter and true bytes."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps}), flush=True)


def bench_summary(args, gdn, gi, inp, q, k, v, g, beta, dev):
    """Times gdn_state_summary / kda_state_summary on the workload (prepare and
    the two state-only passes) and the apply step over its (sequence, head)
    pairs, each call after a 1 GiB read; prints one JSON line."""
    import torch
    B, T, H, K, V = inp.B, inp.T, inp.H, inp.K, inp.V
    N = inp.num_seqs
    kw = dict(q=q, cu_seqlens=inp.cu_seqlens, kda=inp.kda, l2norm_qk=bool(inp.flags & gi.FLAG_L2NORM_QK),
              beta_sigmoid=bool(inp.flags & gi.FLAG_BETA_SIGMOID))
    M, S = gdn.state_summary(k, v, g, beta, **kw)
    need = gdn.lib.gdn_state_summary_workspace_bytes(int(inp.kda), B, T, H, K, V, N, None if inp.cu_seqlens is None
                                                     else np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
                                                     .ctypes.data_as(ctypes.c_void_p))
    ws = torch.empty(int(need), dtype=torch.uint8, device=dev)
    s_in = torch.randn((N, H, K, V), device=dev) * 0.02
    out = torch.empty_like(S)
    scrub = torch.full((max(args.scrub_mib, 1) * (1 << 20) // 4,), 1.0, dtype=torch.float32, device=dev)

    def timed(fn, n):
        ts = []
        for _ in range(n):
            if args.scrub_mib:
                scrub.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))

    summ = lambda: gdn.state_summary(k, v, g, beta, workspace=ws, **kw)
    app = lambda: gdn.state_summary_apply(M, S, s_in, out=out)
    for _ in range(args.warmup):
        summ()
        app()
    torch.cuda.synchronize()
    ms, p10, p90 = timed(summ, args.steps)
    ams, _, _ = timed(app, args.steps)
    tokens = B * T
    kind = "KDA" if inp.kda else "GDN"
    line = {
        "metric": "state summary tokens/s",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "%s state summary (M, S) B=%d T=%d H=%d, %d sequences" % (kind, B, T, H, N),
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": K, "parallelism": "single-gpu"},
        "timing": {"per_call": "median of %d calls, %d MiB read before each" % (args.steps, args.scrub_mib),
                   "p10_ms": round(p10, 5), "p90_ms": round(p90, 5)},
        "apply_us": round(ams * 1e3, 2),
        "apply_pairs": N * H,
    }
    print(json.dumps(line), flush=True)


def bench_bwd(args, gdn, gi, inp, q, k, v, g, beta, dev):
    """Times gdn_chunk_bwd on the workload (forward recompute: prepare and the
    state pass storing h and v_new; then the reverse state pass, the state
    products and the per-chunk gradients), each call after a 1 GiB read;
    prints one JSON line. The cotangents are seeded N(0,1) (dO, bf16) and
    0.1 N(0,1) (dS_final)."""
    import torch
    if inp.kda:
        return bench_kda_bwd(args, gdn, gi, inp, q, k, g, beta, dev)
    B, T, H, K, V = inp.B, inp.T, inp.H, inp.K, inp.V
    N = inp.num_seqs
    gen = torch.Generator(device=dev).manual_seed(7)
    do = torch.randn((B, T, H, V), device=dev, generator=gen).to(torch.bfloat16)
    dsf = torch.randn((N, H, K, V), device=dev, generator=gen) * 0.1
    s0 = None if inp.initial_state is None else torch.from_numpy(inp.initial_state).to(dev)
    cu = None if inp.cu_seqlens is None else np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
    need = gdn.lib.gdn_chunk_bwd_workspace_bytes(B, T, H, K, V, N, None if cu is None else
                                                 cu.ctypes.data_as(ctypes.c_void_p), inp.flags & 3)
    ws = torch.empty(int(need), dtype=torch.uint8, device=dev)
    kw = dict(scale=inp.scale, initial_state=s0, d_final_state=dsf, cu_seqlens=inp.cu_seqlens,
              l2norm_qk=bool(inp.flags & gi.FLAG_L2NORM_QK), beta_sigmoid=bool(inp.flags & gi.FLAG_BETA_SIGMOID),
              workspace=ws)
    call = lambda: gdn.gdn_chunk_bwd(q, k, v, g, beta, do, **kw)
    scrub = torch.full((max(args.scrub_mib, 1) * (1 << 20) // 4,), 1.0, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(args.steps):
        if args.scrub_mib:
            scrub.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    # per-kernel durations from the library's events (a second pass, same protocol)
    gdn.timing_enable(True)
    for _ in range(args.steps):
        if args.scrub_mib:
            scrub.sum()
        call()
    torch.cuda.synchronize()
    kms, ncalls = gdn.bwd_timing_read()
    gdn.timing_enable(False)
    names = ("prepare", "fwd_state", "bwd_dh", "bwd_sprod", "bwd_intra")
    kus = {n: 1e3 * t / max(ncalls, 1) for n, t in zip(names, kms)}
    # algorithmic work per chunk-head of each backward kernel (64 rows)
    cmh = gdn.num_chunks(B, T, inp.cu_seqlens) * H
    work = {
        # bf16 MFMA products of the reverse pass: k dS, Aqk^T dO, T^T dV', q^T dO, k^T Z
        "bwd_dh": ("mfma", 2 * (64 * 128 * 128 + 2 * 64 * 64 * 128 + 2 * 128 * 64 * 128), MFMA_BF16_PEAK_TFLOPS,
                   "gdn_bwd_dh_kernel"),
        # S, dS_next (64 KiB each), dV', V' (32 KiB each), dO (16 KiB) read; E, F, D (96 KiB) written
        "bwd_sprod": ("hbm", 2 * 65536 + 2 * 32768 + 16384 + 98304, HBM_PEAK_GBPS, "gdn_bwd_sprod_kernel"),
        # fp32 MFMA products of the per-chunk gradients (lower tiles only where triangular)
        "bwd_intra": ("mfma", 11206656, MFMA_FP32_PEAK_TFLOPS, "gdn_bwd_intra_kernel"),
    }
    dom = max(work, key=lambda n: kus[n])
    bound, per_cmh, peak, sym = work[dom]
    per_launch = per_cmh * cmh
    if bound == "hbm":
        achieved = per_launch / (kus[dom] * 1e-6) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                "frac": round(achieved / peak, 4)}
    else:
        achieved = per_launch / (kus[dom] * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    roof["traffic"] = recorded_traffic("bwd_" + args.workload, sym)
    tokens = B * T
    line = {
        "metric": "bwd tokens/s (GDN gradients dq dk dv dg dbeta dS0)",
        "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "GDN backward B=%d T=%d H=%d, %d sequences, flags %d" % (B, T, H, N, inp.flags & 3),
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": K, "parallelism": "single-gpu"},
        "roofline": roof,
        "kernels_us": {n: round(v, 2) for n, v in kus.items()},
        "timing": {"per_call": "median of %d calls, %d MiB read before each" % (args.steps, args.scrub_mib),
                   "p10_ms": round(float(np.percentile(ts, 10)), 5),
                   "p90_ms": round(float(np.percentile(ts, 90)), 5)},
    }
    print(json.dumps(line), flush=True)


# Reverse state pass of the KDA backward, flops per (chunk, head): dV' = KG dS
# (64x128x128) + Aqk^T dO (lower triangle, 2080 x 128), Y = T^T dV' (2080 x
# 128), dS update QD^T dO + KDB^T Y (2 x 128x64x128) and the decay. The
# products run on the fp32 matrix instruction, so they are priced against
# the fp32 matrix peak.
KDA_DH_FLOPS = 2 * (64 * 128 * 128 + 2080 * 128 + 2080 * 128 + 2 * 128 * 64 * 128) + 128 * 128


def bench_kda_bwd(args, gdn, gi, inp, q, k, g, beta, dev):
    """Times kda_chunk_bwd (the whole KDA backward, the headline), its stage
    kda_bwd_state_pass (prepare, then the reverse state pass) and the prepare
    alone (stage entry), each call after a 1 GiB read; the reverse pass is the
    difference of the last two. Prints one JSON line."""
    import torch
    B, T, H, K, V = inp.B, inp.T, inp.H, inp.K, inp.V
    N = inp.num_seqs
    gen = torch.Generator(device=dev).manual_seed(7)
    do = torch.randn((B, T, H, V), device=dev, generator=gen).to(torch.bfloat16)
    dsf = torch.randn((N, H, K, V), device=dev, generator=gen) * 0.1
    cu = None if inp.cu_seqlens is None else np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.c_void_p)
    flags = inp.flags & 3
    need = gdn.lib.kda_bwd_state_pass_workspace_bytes(B, T, H, K, V, N, cu_p, flags)
    ws = torch.empty(int(need), dtype=torch.uint8, device=dev)
    NT = gdn.num_chunks(B, T, inp.cu_seqlens)
    dh = torch.empty((H, NT, K, V), dtype=torch.float32, device=dev)
    dvn = torch.empty((H, NT, 64, V), dtype=torch.float32, device=dev)
    ds0 = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    tm = torch.empty((H, NT, 64, 128), dtype=torch.bfloat16, device=dev)
    aq = torch.empty((H, NT, 64, 64), dtype=torch.bfloat16, device=dev)
    vec = torch.empty((H, NT, 8, 64), dtype=torch.float32, device=dev)
    gk = torch.empty((H, NT, 64, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)

    need_all = gdn.lib.kda_chunk_bwd_workspace_bytes(B, T, H, K, V, N, cu_p, flags)
    ws_all = torch.empty(int(need_all), dtype=torch.uint8, device=dev)
    grads = [torch.empty((B, T, H, K), dtype=torch.float32, device=dev) for _ in range(4)]
    dbeta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    v = torch.from_numpy(inp.v).view(torch.bfloat16).to(dev)

    def backward():
        rc = gdn.lib.kda_chunk_bwd(P(q), P(k), P(v), P(g), P(beta), None, cu_p, N, B, T, H, K, V, float(inp.scale),
                                   flags, P(do), P(dsf), *[P(t) for t in grads], P(dbeta), P(ds0), P(ws_all),
                                   int(need_all), sp)
        if rc != 0:
            raise RuntimeError(gdn.last_error())

    def whole():
        rc = gdn.lib.kda_bwd_state_pass(P(q), P(k), P(g), P(beta), cu_p, N, B, T, H, K, V, float(inp.scale), flags,
                                        P(do), P(dsf), P(dh), P(dvn), P(ds0), P(ws), int(need), sp)
        if rc != 0:
            raise RuntimeError(gdn.last_error())

    def prepare():
        rc = gdn.lib.gdn_stage_prepare(1, P(q), P(k), P(g), P(beta), cu_p, N, B, T, H, K, V, float(inp.scale), flags,
                                       P(tm), P(aq), P(vec), P(gk), sp)
        if rc != 0:
            raise RuntimeError(gdn.last_error())

    scrub = torch.full((max(args.scrub_mib, 1) * (1 << 20) // 4,), 1.0, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            if args.scrub_mib:
                scrub.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    bwd_ms = timed(backward)
    ms = timed(whole)
    prep_ms = timed(prepare)
    dh_ms = ms - prep_ms
    flops = NT * H * KDA_DH_FLOPS
    achieved = flops / (dh_ms * 1e-3) / 1e12
    tokens = B * T
    line = {
        "metric": "KDA backward tokens/s", "value": round(tokens / (bwd_ms * 1e-3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(bwd_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "KDA backward (kda_chunk_bwd) B=%d T=%d H=%d, %d sequences" % (B, T, H, N),
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": K,
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": "kda_bwd_dh", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_FP32_PEAK_TFLOPS, 4), "traffic": None},
        "kernels_us": {"prepare": round(prep_ms * 1e3, 2), "reverse_state_pass": round(dh_ms * 1e3, 2),
                       "recompute_products_and_per_chunk": round((bwd_ms - ms) * 1e3, 2)},
        "timing": {"per_call": "median of %d calls, %d MiB read before each; reverse pass = "
                               "kda_bwd_state_pass - prepare alone, rest = kda_chunk_bwd - kda_bwd_state_pass"
                               % (args.steps, args.scrub_mib)},
    }
    print(json.dumps(line), flush=True)


def bench_conv(args, gdn, gi, dev):
    """Times gdn_short_conv on the projections of the workload's GDN layer:
    D = 3 * H * 128 channels (q, k, v), W = 4, SiLU, each call after a 1 GiB
    read; HBM-bound, so reported against the HBM roofline (algorithmic bytes:
    x read once, y written once)."""
    import torch
    B, T, H = gi.WORKLOADS[args.workload][:3]
    D = 3 * H * 128
    inp = gi.make_conv_inputs(B, T, D, W=4, seed=2001)
    x = torch.from_numpy(inp.x).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(inp.weight).to(dev)
    y = torch.empty_like(x)
    scrub = torch.full((max(args.scrub_mib, 1) * (1 << 20) // 4,), 1.0, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        gdn.short_conv(x, w, out=y)
    ts = []
    for _ in range(args.steps):
        if args.scrub_mib:
            scrub.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gdn.short_conv(x, w, out=y)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    alg = 2.0 * B * T * D * 2
    gbps = alg / (ms * 1e-3) / 1e9
    line = {
        "metric": "short conv tokens/s", "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "causal depthwise Conv1d + SiLU, B=%d T=%d D=%d W=4" % (B, T, D), "global_batch": B,
                   "seq_len": T, "channels": D, "parallelism": "single-gpu"},
        "roofline": {"kernel": "short_conv", "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
        "timing": {"per_call": "median of %d calls, %d MiB read before each" % (args.steps, args.scrub_mib),
                   "p10_ms": round(float(np.percentile(ts, 10)), 5), "p90_ms": round(float(np.percentile(ts, 90)), 5)},
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the forward pass is benchmarked on a single MI355X "
              "(--gpus %d / WORLD_SIZE %d refused)." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import chunked_gated_delta_03_amd as gdn
    import gdn_inputs as gi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "conv":
        bench_conv(args, gdn, gi, dev)
        return
    inp = gi.make_inputs(args.workload)
    B, T, H, K, V = inp.B, inp.T, inp.H, inp.K, inp.V
    N = inp.num_seqs
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
    q, k, v, beta = bf(inp.q), bf(inp.k), bf(inp.v), bf(inp.beta)
    g = torch.from_numpy(inp.g).to(dev)
    s0 = None if inp.initial_state is None else torch.from_numpy(inp.initial_state).to(dev)
    o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    ws_bytes = gdn.workspace_bytes(B, T, H, cu_seqlens=inp.cu_seqlens, kda=inp.kda, flags=inp.flags)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    cu = None if inp.cu_seqlens is None else np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
    cu_p = None if cu is None else cu.ctypes.data_as(ctypes.c_void_p)
    if args.op == "summary":
        bench_summary(args, gdn, gi, inp, q, k, v, g, beta, dev)
        return
    if args.op == "bwd":
        bench_bwd(args, gdn, gi, inp, q, k, v, g, beta, dev)
        return
    stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    if args.gate_in_kernel:
        if inp.gate_raw is None:
            raise SystemExit("--gate-in-kernel: the %s workload has no raw gate" % args.workload)
        g_raw = torch.from_numpy(inp.gate_raw).to(dev)
        a_log = torch.from_numpy(inp.A_log).to(dev)
        dt_bias = torch.from_numpy(inp.dt_bias).to(dev)
        fn = gdn.lib.kda_chunk_fwd_gated if inp.kda else gdn.lib.gdn_chunk_fwd_gated
        call_args = (P(q), P(k), P(v), P(g_raw), P(a_log), P(dt_bias), P(beta), P(s0), cu_p, N, B, T, H, K, V,
                     float(inp.scale), int(inp.flags), P(o), P(fs), P(ws), ws_bytes,
                     ctypes.c_void_p(stream.cuda_stream))
    else:
        fn = gdn.lib.kda_chunk_fwd if inp.kda else gdn.lib.gdn_chunk_fwd
        call_args = (P(q), P(k), P(v), P(g), P(beta), P(s0), cu_p, N, B, T, H, K, V, float(inp.scale),
                     int(inp.flags), P(o), P(fs), P(ws), ws_bytes, ctypes.c_void_p(stream.cuda_stream))

    def step():
        rc = fn(*call_args)
        if rc != 0:
            raise RuntimeError("gdn call failed: %s" % gdn.last_error())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # scrubbed: one event pair per call, a 1 GiB read before each
    scrub = torch.full((max(args.scrub_mib, 1) * (1 << 20) // 4,), 1.0, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def scrub_read():
        if args.scrub_mib:
            scrub.sum()

    def timed_calls(before):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            before(i)
            evs[i][0].record(stream)
            step()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    per_call = timed_calls(lambda i: scrub_read())

    # scrubbed again, with per-kernel events recorded by the library
    gdn.timing_enable(True)
    gdn.timing_read()
    for i in range(args.steps):
        scrub_read()
        step()
    torch.cuda.synchronize()
    gdn.timing_enable(False)
    prep_ms, state_ms, calls = gdn.timing_read()
    assert calls == args.steps

    # the buffer written instead of read before each call
    per_call_dirty = timed_calls(lambda i: scrub.fill_(float(i)) if args.scrub_mib else None)
    del scrub

    # warm: the same number of calls back to back
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    warm_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    wall_ms_per_step = (t1 - t0) * 1e3 / args.steps

    # host side of one call (argument checks, for packed input the chunk
    # table build and its upload, the launches), the GPU drained before each
    host_us = []
    for _ in range(args.steps):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        step()
        host_us.append((time.perf_counter() - h0) * 1e6)
    torch.cuda.synchronize()

    ms_per_step = float(np.median(per_call))
    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)
    th = tokens * H
    prep_us = prep_ms * 1e3 / calls
    state_us = state_ms * 1e3 / calls

    n_states = (1 if inp.flags & gi.FLAG_OUTPUT_FINAL_STATE else 0) + (0 if s0 is None else 1)
    prep_bytes = th * (KDA_PREP_BYTES if inp.kda else GDN_PREP_BYTES)
    state_bytes = th * STATE_BYTES + n_states * N * H * STATE_BYTES_PER_UNIT
    path_bytes = prep_bytes + state_bytes
    kernels = {
        "prepare": {"avg_us": prep_us, "alg_bytes": prep_bytes, "symbol": "prepare_kernel"},
        "state_output": {"avg_us": state_us, "alg_bytes": state_bytes, "symbol": "kda_state_kernel" if inp.kda else "gdn_state_kernel"},
    }
    dom_name = max(kernels, key=lambda n: kernels[n]["avg_us"])
    dom = kernels[dom_name]
    # achieved: the call's algorithmic bytes (1,030 B per token-head, 1,538 for
    # KDA, plus 64 KiB per state read or written) over the dominant kernel's
    # average duration; the same kernel's share of those bytes by first touch
    # is reported beside it
    achieved = path_bytes / (dom["avg_us"] * 1e-6) / 1e9
    achieved_ft = dom["alg_bytes"] / (dom["avg_us"] * 1e-6) / 1e9
    roofline = {
        "kernel": dom_name,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": None if args.gate_in_kernel else recorded_traffic(args.workload, dom["symbol"]),
        "alg_bytes": int(path_bytes),
        "mfma_busy": None if args.gate_in_kernel else recorded_mfma(args.workload, dom["symbol"]),
        "first_touch": {"alg_bytes": int(dom["alg_bytes"]), "achieved": round(achieved_ft, 1),
                        "frac": round(achieved_ft / HBM_PEAK_GBPS, 4)},
    }
    path_gbps = path_bytes / (ms_per_step * 1e-3) / 1e9
    mfma_frac = th * ALG_FLOPS_PER_TH / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFLOPS * 1e12)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        units = [(n, h) for n in range(N) for h in range(H)]
        sample_desc = "whole workload"
        budget_units = len(units)
        if args.workload in ("long", "kda"):
            budget_units = 8 if args.workload == "long" else 16
            units = units[:budget_units]
            sample_desc = "%d of %d (sequence, head) units" % (budget_units, N * H)
        tok_units = sum((int(inp.cu_seqlens[n + 1] - inp.cu_seqlens[n]) if inp.cu_seqlens is not None else T)
                        for n, _ in units)
        # repeat the sample until about 10 s of CPU time has been measured
        reps = 0
        c0 = time.perf_counter()
        while True:
            oracle.recur(inp, units=units)
            reps += 1
            if time.perf_counter() - c0 >= 10.0 or reps >= 50:
                break
        c1 = time.perf_counter()
        per = (c1 - c0) / reps
        cpu = {
            "value": round(tok_units / H / per, 1),
            "unit": "tokens/s",
            "cores": oracle.num_threads(),
            "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": "fp64 token recurrence (C, OpenMP over units) on %s: %d token-heads, %.3f s per pass, "
                      "%d passes; tokens/s = token-heads / H / s" % (sample_desc, tok_units, per, reps),
        }

    wl = {
        "gdn": "GDN B=4 T=4096 H=16 K=V=128 chunk 64, in-kernel L2-norm + sigmoid(beta), final state",
        "varlen": "packed GDN B=1 T=32768 H=16 docs~U[17,8192], per-doc initial/final state",
        "long": "GDN B=1 T=131072 H=32 K=V=128 chunk 64",
        "kda": "KDA B=2 T=8192 H=32 K=V=128 per-channel log2 gate",
        "tiny": "GDN B=1 T=256 H=2",
    }[args.workload]
    if args.gate_in_kernel:
        wl += ", gate -exp(A_log) softplus(x + dt_bias) formed in the kernel"
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "global_batch": B, "seq_len": T, "heads": H, "head_dim": K,
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "mfma_bf16_frac": round(mfma_frac, 4),
        "path_alg_hbm_frac": round(path_gbps / HBM_PEAK_GBPS, 4),
        "kernels_us": {"prepare": round(prep_us, 2), "state_output": round(state_us, 2)},
        "timing": {"per_call": "median of %d calls, %d MiB read before each" % (args.steps, args.scrub_mib),
                   "p10_ms": round(float(np.percentile(per_call, 10)), 5),
                   "p90_ms": round(float(np.percentile(per_call, 90)), 5),
                   "written_scrub_ms": round(float(np.median(per_call_dirty)), 5),
                   "warm_ms_per_step": round(warm_ms_per_step, 5),
                   "warm_tokens_per_s": round(tokens / (warm_ms_per_step * 1e-3), 1),
                   "host_call_us": round(float(np.median(host_us)), 1)},
        "wall_ms_per_step": round(wall_ms_per_step, 5),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
