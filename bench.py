#!/usr/bin/env python3
"""Benchmark of the four-direction Hope memory scan on one MI355X.

One step = one hope_scan2d_forward call over the whole batch of the stage-3
workload (B=128, 14x14 map, D=384 as 6 heads of 64, row/column chunks of 14,
bf16 inputs, fp32 state), inputs already resident in HBM.  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload IDX] [--no-cpu-baseline]
                  [--copy-probe-mib N] [--readout running] [--variants ...] [--backward]
                  [--block] [--exports]

--backward times the gradient pass (hope_scan2d_backward) instead, as its own JSON line.

Warm-up is W untimed steps and, beyond them, as many more as it takes to keep the GPU
busy for 0.2 s, so that the clock has settled before the K timed steps.

The roofline object is that of the scan kernel: its time per launch comes from HIP
events the library records around that kernel alone (the route sum that follows it
is excluded), on the stream the call is enqueued on.  "traffic" is the scan kernel's
HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE counter runs, scaled by
what the same counters read for a plain device copy of known size (--copy-probe-mib
runs one after the timed steps); it is read from the committed record under
profiles/ and reported only while the kernel sources hash to the recorded value.

Roofline of the scan kernel: algorithmic work per (token, head, route), in
multiply-accumulates, is 4d^2 + 2d for the projections and the readout (bf16
inputs, MFMA class, 2.5 PFLOP/s) plus the cheapest exact fp32 chunk form for the
gain and the carry, min(F1, F2, F3) (fp32 class, 157.3 TFLOP/s):
  F1 = 3d^2 + (4d^3 + 2d^2)/C,  F2 = Cd + C^2/6 + d^2 + (4d^3 + 2d^2)/C,
  F3 = Cd + C^2/6 + 8d^2 + 4d.
The roofline time is the sum of each class's flops over its peak; "peak" in the
JSON is the total flop count over that time (the blend of the two peaks), so
frac = roofline time / measured kernel time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

PEAK_BF16 = 2.5e15      # dense bf16 MFMA, FLOP/s
PEAK_FP32 = 157.3e12    # fp32 matrix / vector, FLOP/s
PEAK_HBM = 8.0e12       # bytes/s
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "scan_traffic.json")
KERNEL_SOURCES = ["chain_mfma.hip", "chain_chunk.hip", "chain_kernel.hip", "mfma_ops.h", "device_common.h", "kernels.h"]
METRIC = wl_metric = "scan tokens/s (positions×dirs) for 4-dir Hope memory scan; % MFMA/HBM peak"


def work_per_token(d: int, C: int, readout: str = "boundary") -> tuple[float, float]:
    """(bf16-class MACs, fp32-class MACs) per (token, head, route).

    The running readout adds, per token, one d x d product of the chunk-start M_mem with
    a write vector (or of G_{t-1} with q_t) and a causal C-long weighting: d^2 + C d / 2.
    """
    bf16 = 4 * d * d + 2 * d
    f1 = 3 * d * d + (4 * d ** 3 + 2 * d * d) / C
    f2 = C * d + C * C / 6 + d * d + (4 * d ** 3 + 2 * d * d) / C
    f3 = C * d + C * C / 6 + 8 * d * d + 4 * d
    extra = d * d + C * d / 2 if readout == "running" else 0.0
    return float(bf16), float(min(f1, f2, f3) + extra)


def roofline_numbers(w: wl.Workload, n_dirs: int = 4, readout: str = "boundary") -> dict:
    d = w.d
    units = w.scan_tokens(n_dirs) * w.n_heads
    f_bf16 = f_fp32 = 0.0
    for C in (w.chunk or w.W, w.chunk or w.H):  # row routes, column routes: half the units each
        bf16, fp32 = work_per_token(d, min(C, w.H * w.W), readout)
        f_bf16 += bf16 * units  # 2 flops per MAC over half the units
        f_fp32 += fp32 * units
    t_compute = f_bf16 / PEAK_BF16 + f_fp32 / PEAK_FP32
    x_bytes = w.B * w.H * w.W * w.D * (2 if w.dtype == "bf16" else 4)
    out_bytes = w.B * w.H * w.W * w.D * 4
    init_bytes = 4 * w.n_heads * w.state_size * 4
    hbm = x_bytes + out_bytes + init_bytes
    # the same work at the bf16 matrix peak as the MFMA kernels execute it: the projections
    # as two bf16 products (x is exact bf16, the state split hi + lo), the readout
    # (d^2 of the bf16-class MACs) and every fp32-class product as three (hi*hi + hi*lo + lo*hi)
    f_read = 2.0 * d * d * units
    t_exec = (2 * (f_bf16 - f_read) + 3 * f_read + 3 * f_fp32) / PEAK_BF16
    return {"flops": f_bf16 + f_fp32, "flops_bf16": f_bf16, "flops_fp32": f_fp32,
            "t_compute": t_compute, "t_as_executed": t_exec, "hbm_bytes": hbm,
            "t_hbm": hbm / PEAK_HBM}


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "self_modifying_memory_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(w: wl.Workload):
    """HBM bytes per scan launch from the counter record, or None when the record is
    missing, has no entry for this workload, or predates the current kernel sources."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)["records"].get(w.name)
    except (OSError, ValueError, KeyError, AttributeError):
        return None
    if not rec or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return float(rec["traffic_bytes_per_launch"])


HOST_WORKERS_MAX = 16  # the GPU machine's CPU share for one GPU


def _oracle_part(args) -> float:
    """One host worker of the CPU baseline: the oracle, as it stands, on a slice of
    (image, head) chains; returns its own busy time."""
    x, init, n_heads, heads, readout, chunk = args
    import oracle
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.scan2d(x, init, n_heads, heads=heads, readout=readout, chunk=chunk)
        return time.perf_counter() - t0


def cpu_baseline(w: wl.Workload, inp: dict, budget_s: float = 15.0, readout: str = "boundary") -> dict:
    """Time the fp64 oracle, as it stands, on a bounded sample of the same workload, split
    over the host cores by (image, head) with one process and one BLAS thread per core."""
    import multiprocessing as mp
    cores = max(1, min(len(os.sched_getaffinity(0)), HOST_WORKERS_MAX))
    # probe: one (image, head) chain set on one core
    probe = _oracle_part((inp["x"][:1], inp["init"], w.n_heads, [0], readout, w.chunk))
    per_core = max(1, int(budget_s / max(probe, 1e-3)))
    units = [(b, h) for b in range(w.B) for h in range(w.n_heads)][:per_core * cores]
    jobs = []
    for c in range(cores):
        mine = units[c::cores]
        if not mine:
            continue
        imgs = sorted({b for b, _ in mine})
        for b in imgs:  # one job per (image, its heads on this core)
            hs = [h for bb, h in mine if bb == b]
            jobs.append((c, (inp["x"][b:b + 1], inp["init"], w.n_heads, hs, readout, w.chunk)))
    ctx = mp.get_context("spawn")  # fresh interpreters: nothing of this process's GPU state
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_part, [(inp["x"][:1, :2, :2], inp["init"], w.n_heads, [0], readout, 0)] * cores)
        t0 = time.perf_counter()
        pool.map(_oracle_part, [j for _, j in jobs], chunksize=1)
        dt = time.perf_counter() - t0
    toks = len(units) * w.H * w.W * 4 / w.n_heads
    return {"value": toks / dt, "unit": "scan tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(units)} of {w.B * w.n_heads} (image, head) chain sets, 4 routes each "
                      f"({toks:.0f} scan-token equivalents) in {dt:.1f} s wall on {cores} worker "
                      f"processes (fp64 numpy, 1 BLAS thread each)"}


def cpu_baseline_backward(w: wl.Workload, inp: dict, g: np.ndarray, budget_s: float = 15.0,
                          readout: str = "boundary") -> dict:
    """Time the gradient oracle (autograd of the fp64 forward), as it stands, on a bounded
    sample of the first image: its first rows (all of them, and then more heads, when the
    whole map fits the budget), one head, all four routes; the column routes of a crop run
    over the crop's height.  A first pass on four rows sizes the sample."""
    import torch as _torch
    from oracle import hope_backward as hb
    threads = _torch.get_num_threads()
    _torch.set_num_threads(1)
    d = w.d

    def run(rows, nh):
        hb.scan2d_backward(inp["x"][:1, :rows, :, :nh * d], inp["init"][:, :nh], nh,
                           g[:1, :rows, :, :nh * d], chunk=w.chunk, readout=readout)

    try:
        r0 = min(w.H, 4)
        t0 = time.perf_counter()
        run(r0, 1)
        t1 = max(time.perf_counter() - t0, 1e-3)
        rows = max(1, min(w.H, int(r0 * budget_s / t1)))
        nh = 1
        if rows == w.H:
            nh = max(1, min(w.n_heads, int(budget_s / (t1 * w.H / r0))))
        t0 = time.perf_counter()
        run(rows, nh)
        dt = time.perf_counter() - t0
    finally:
        _torch.set_num_threads(threads)
    toks = rows * w.W * 4 * nh
    return {"value": toks / dt, "unit": "scan tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"1 of {w.B} images, its first {rows} of {w.H} rows, {nh} of {w.n_heads} heads, "
                      f"4 routes ({toks} scan-token equivalents) in {dt:.1f} s, torch fp64 autograd, 1 thread"}


def run_backward(args, w: wl.Workload, inp: dict, x_host, dev) -> int:
    """The backward pass (hope_scan2d_backward) as the timed step.  Roofline: the gradient
    of every forward product costs two products of the same size and the forward is
    recomputed once, so the algorithmic work is 3x the forward's.  At d = 32 (any chunk
    length, in 16-token blocks) and at d = 64 with chunks of at most 16 tokens the kernel
    runs its products on the fp32 matrix cores (the rest on the vector ALUs); the whole of
    it is charged at the fp32 peak (157.3 TFLOP/s, matrix and vector alike)."""
    import torch
    from self_modifying_memory_amd.scan2d import (hope_scan2d_backward,
                                                  hope_scan2d_backward_workspace_size)
    x = x_host.to(dev)
    init = torch.from_numpy(inp["init"].copy()).to(dev)
    g_np = np.random.Generator(np.random.PCG64(7)).standard_normal(
        (w.B, w.H, w.W, w.D)).astype(np.float32)
    g = torch.from_numpy(g_np).to(dev)
    ws = torch.empty(max(256, hope_scan2d_backward_workspace_size(x, w.n_heads, 15, w.chunk)),
                     dtype=torch.uint8, device=dev)
    gx = torch.empty(x.shape, dtype=torch.float32, device=dev)
    gi = torch.empty_like(init)
    stream = torch.cuda.current_stream()

    def step():
        hope_scan2d_backward(x, init, w.n_heads, g, 15, w.chunk, stream=stream, grad_x=gx,
                             grad_init=gi, workspace=ws, readout=args.readout)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.2:  # clock settling, untimed
        step()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    c_avg = float(np.mean(call_ms)) * 1e-3
    roof = roofline_numbers(w, readout=args.readout)
    flops = 3 * roof["flops"]
    wy = w.d == 64 and max(w.chunk or w.W, w.chunk or w.H) <= 16
    kname = ("chain_backward_wy_kernel" if wy else
             "chain_backward_wy32_kernel" if w.d == 32 else "chain_backward_kernel")
    wy = wy or w.d == 32
    rec = {
        "metric": "backward scan tokens/s (positions x dirs): gradients of the 4-dir Hope memory "
                  "scan with respect to the map and the initial memories",
        "value": w.scan_tokens(4) * args.steps / wall,
        "unit": "scan tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "W": w.W, "D": w.D,
                   "n_heads": w.n_heads, "chunk": w.chunk or w.W, "dirs": 4, "x_dtype": w.dtype,
                   "pass": "backward", "readout": args.readout},
        "roofline": {"bound": "mfma" if wy else "alu", "achieved": flops / c_avg / 1e12,
                     "peak": PEAK_FP32 / 1e12,
                     "unit": "TFLOP/s", "frac": flops / c_avg / PEAK_FP32, "traffic": None,
                     "kernel": kname + " (with the gradient reduction and route sum)",
                     "kernel_ms": c_avg * 1e3, "kernel_ms_median": float(np.median(call_ms)),
                     "kernel_ms_p10_p90": [float(np.percentile(call_ms, 10)),
                                           float(np.percentile(call_ms, 90))],
                     "calls_timed": len(call_ms)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_backward(w, inp, g_np.astype(np.float64), readout=args.readout)
    print(json.dumps(rec), flush=True)
    return 0


def run_block(args, w: wl.Workload, dev) -> int:
    """One VisionHOPE block (hope_block_forward: positional encoding, LayerNorms, the five
    projections, the depthwise branches, the operator and the FFN) on the workload's shape
    with synthetic weights, as the timed step, in the pages' evaluated form (VisionHOPE
    App. C.3: inner width D_m = D / 2, D / 32 heads of 16; --block-inner full keeps D_m = D
    with the workload's heads).  Roofline: the projections' flops at the bf16 matrix peak
    plus the operator's at its own kernel's bound; the depthwise and LayerNorm passes are
    left out of the count."""
    import dataclasses
    import torch
    from self_modifying_memory_amd import _native as N
    from self_modifying_memory_amd.block import hope_block_forward, hope_block_workspace_size
    from self_modifying_memory_amd.scan2d import hope_scan2d_kernel_name
    F = 4 * w.D
    Dm, nh = (w.D, w.n_heads) if args.block_inner == "full" else (w.D // 2, w.D // 32)
    op = dataclasses.replace(w, D=Dm, n_heads=nh)
    rng = np.random.Generator(np.random.PCG64(31))
    x_np = rng.standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32)
    wts = wl.draw_block_weights(w.D, nh, F, seed=32, D_m=Dm)
    names = {"init_memories": "init", "route_scales": "scales"}
    wd = {}
    for name in N.BLOCK_WEIGHT_FIELDS:
        key = names.get(name, name)
        if key + "_bits" in wts:
            wd[name] = torch.from_numpy(wts[key + "_bits"].view(np.int16).copy()).view(torch.bfloat16).to(dev)
        else:
            wd[name] = torch.from_numpy(np.ascontiguousarray(wts[key], dtype=np.float32)).to(dev)
    x = torch.from_numpy(x_np).to(dev)
    out = torch.empty_like(x)
    ws = torch.empty(hope_block_workspace_size(w.B, w.H, w.W, w.D, nh, F, w.chunk, Dm),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    zq = torch.empty((w.B, w.H, w.W, Dm), dtype=torch.bfloat16, device=dev)
    kname = hope_scan2d_kernel_name(zq, nh, 15, w.chunk, queries=torch.empty_like(zq, dtype=torch.float32),
                                    skip=wd["skip"], route_scales=wd["route_scales"])
    del zq

    def step():
        hope_block_forward(x, wd, nh, F, w.chunk, D_m=Dm, out=out, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.2:  # clock settling, untimed
        step()
        torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    c_avg = float(np.mean(call_ms)) * 1e-3
    M = w.B * w.H * w.W
    f_gemm = 2.0 * M * (2 * w.D * Dm + Dm * Dm + 2 * w.D * F)
    roof = roofline_numbers(op)
    on_mfma = kname != "chain_kernel"
    t_op = roof["t_compute"] if on_mfma else roof["flops"] / PEAK_FP32
    t_roof = f_gemm / PEAK_BF16 + t_op
    rec = {
        "metric": "block pixels/s: one VisionHOPE block (Eq. 27, App. B.5) per pixel of the map",
        "value": M * args.steps / wall, "unit": "pixels/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_block", "B": w.B, "H": w.H, "W": w.W, "D": w.D,
                   "D_m": Dm, "n_heads": nh, "d": Dm // nh, "ffn_dim": F,
                   "chunk": w.chunk or w.W, "dirs": 4},
        "roofline": {"bound": "mfma", "achieved": (f_gemm + roof["flops"]) / c_avg / 1e12,
                     "peak": (f_gemm + roof["flops"]) / t_roof / 1e12, "unit": "TFLOP/s",
                     "frac": t_roof / c_avg, "traffic": None,
                     "kernel": "whole block call (projections at the bf16 peak, 2.5 PFLOP/s; the "
                               f"operator ({kname}) at its own bound)",
                     "operator_kernel": kname,
                     "kernel_ms": c_avg * 1e3, "kernel_ms_median": float(np.median(call_ms)),
                     "t_roof_ms": t_roof * 1e3,
                     "kernel_ms_p10_p90": [float(np.percentile(call_ms, 10)),
                                           float(np.percentile(call_ms, 90))],
                     "calls_timed": len(call_ms)},
    }
    if not args.no_cpu_baseline:
        from oracle import hope_block as hbk
        ow = {k: v.astype(np.float64) for k, v in wts.items() if not k.endswith("_bits")}
        t0 = time.perf_counter()
        hbk.block_forward(x_np[:1], ow, nh, chunk=w.chunk)
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": w.H * w.W / dt, "unit": "pixels/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"1 of {w.B} images ({w.H * w.W} pixels) in {dt:.1f} s, "
                                         f"fp64 numpy"}
    print(json.dumps(rec), flush=True)
    return 0


def run_exports(args, w: wl.Workload, x_host, dev) -> int:
    """The gather and merge exports alone (hope_debug_cross_scan: the map into the four
    route orders; hope_debug_cross_merge: the four route sequences summed back into place,
    fp32), one pair per step on the workload's map.  Both are pure data movement, so the
    roofline is HBM: algorithmic bytes = the map read once and four route copies written
    (scan), four route copies read and the fp32 map written (merge)."""
    import torch
    from self_modifying_memory_amd.scan2d import hope_debug_cross_merge, hope_debug_cross_scan
    x = x_host.to(dev)
    es = x.element_size()
    n = w.B * w.H * w.W * w.D
    routes = torch.empty((4, w.B, w.H * w.W, w.D), dtype=x.dtype, device=dev)
    out = torch.empty((w.B, w.H, w.W, w.D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup)):
        hope_debug_cross_scan(x, 15, routes, stream=stream)
        hope_debug_cross_merge(routes, w.H, w.W, 15, out, stream=stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        hope_debug_cross_scan(x, 15, routes, stream=stream)
        e[1].record(stream)
        hope_debug_cross_merge(routes, w.H, w.W, 15, out, stream=stream)
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_scan = float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    t_merge = float(np.median([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    b_scan = n * es * 5
    b_merge = n * es * 4 + n * 4
    step_s = wall / args.steps
    rec = {
        "metric": "scan tokens/s through the gather and merge exports (cross-scan + cross-merge)",
        "value": w.B * w.H * w.W * 4 / step_s, "unit": "scan tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if es == 2 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "W": w.W, "D": w.D, "dirs": 4,
                   "path": "exports"},
        "roofline": {"bound": "hbm", "achieved": b_merge / t_merge / 1e9, "peak": 8000.0,
                     "unit": "GB/s", "frac": b_merge / t_merge / 8e12, "traffic": None,
                     "kernel": "cross_merge_vec_kernel", "kernel_ms": t_merge * 1e3,
                     "cross_scan_ms": t_scan * 1e3, "cross_scan_GBps": b_scan / t_scan / 1e9,
                     "cross_scan_frac": b_scan / t_scan / 8e12},
    }
    if not args.no_cpu_baseline:
        import oracle
        xs = x_host.float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 2.0:
            seqs = {r: oracle.cross_scan(xs, r) for r in range(4)}
            oracle.cross_merge(seqs, w.H, w.W)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        rec["cpu_baseline"] = {"value": w.B * w.H * w.W * 4 / dt, "unit": "scan tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the whole map, {reps} passes in {dt * reps:.1f} s, numpy"}
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--sets", type=int, default=5, help="rotated input/output buffer sets")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--readout", choices=["boundary", "running"], default="boundary",
                    help="readout memory inside a chunk (the default is the chunk-start one)")
    ap.add_argument("--variants", default="",
                    help="comma-separated VisionHOPE variants to enable together: scales, skip, "
                         "counts, hard_injection, soft_spectral, frozen_kv, frozen_dynamics, "
                         "no_dgd, queries (synthetic scales / skip / queries)")
    ap.add_argument("--mem-chunk", type=int, default=0,
                    help="two chunk sizes: the working memory's boundary every this many tokens "
                         "(0: one chunk size)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gradients) instead of the forward scan")
    ap.add_argument("--block", action="store_true",
                    help="time one VisionHOPE block around the scan instead of the scan alone")
    ap.add_argument("--block-inner", choices=["half", "full"], default="half",
                    help="the block's inner width: D/2 with heads of 16 (the pages' evaluated "
                         "models) or D with the workload's heads")
    ap.add_argument("--exports", action="store_true",
                    help="time the gather / merge exports (cross-scan, cross-merge) alone")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: every (image, head, route) chain of this scan is "
              "independent, so more GPUs would only split the batch; run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from self_modifying_memory_amd.scan2d import (alloc_workspace, hope_scan2d_forward,
                                                  hope_scan2d_kernel_name)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    w = wl.WORKLOADS[args.workload]
    inp = wl.draw_workload(w, live=True)
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        x_host = torch.from_numpy(inp["x_bits"].view(np.int16).copy()).view(torch.bfloat16)
    else:
        x_host = torch.from_numpy(inp["x"].copy())
    if args.backward:
        return run_backward(args, w, inp, x_host, dev)
    if args.block:
        return run_block(args, w, dev)
    if args.exports:
        return run_exports(args, w, x_host, dev)
    init = torch.from_numpy(inp["init"].copy()).to(dev)
    sets = []
    for _ in range(max(1, args.sets)):
        x = x_host.to(dev)
        sets.append((x, torch.empty(x.shape, dtype=torch.float32, device=dev),
                     alloc_workspace(x, w.n_heads, 15, w.chunk)))
    stream = torch.cuda.current_stream()
    var = [v for v in args.variants.split(",") if v]
    known = {"scales", "skip", "counts", "hard_injection", "soft_spectral", "frozen_kv",
             "frozen_dynamics", "no_dgd", "queries"}
    if set(var) - known:
        print(f"unknown variants {sorted(set(var) - known)}", file=sys.stderr)
        return 2
    vkw = {}
    vrng = np.random.Generator(np.random.PCG64(123))
    if "scales" in var:
        vkw["route_scales"] = torch.from_numpy(vrng.uniform(0.5, 1.5, (4, w.D)).astype(np.float32)).to(dev)
    if "skip" in var:
        vkw["skip"] = torch.from_numpy((vrng.standard_normal(w.D) * 0.3).astype(np.float32)).to(dev)
    if "counts" in var:
        vkw["counts"] = torch.zeros(3, dtype=torch.int64, device=dev)
    if "hard_injection" in var:
        vkw["injection"] = "hard"
    if "soft_spectral" in var:
        vkw["spectral"] = "soft"
    frozen = [f for f, name in (("kv", "frozen_kv"), ("dynamics", "frozen_dynamics")) if name in var]
    if frozen:
        vkw["frozen"] = tuple(frozen)
    if "no_dgd" in var:
        vkw["no_dgd"] = True
    if "queries" in var:
        vkw["queries"] = torch.from_numpy(vrng.standard_normal((w.B, w.H, w.W, w.D)).astype(np.float32)).to(
            dev).to(x_host.dtype)
    # events around the scan kernel alone, recorded by the library on this stream
    scan_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    for a, b in scan_ev:
        a.record(stream)
        b.record(stream)

    def step(i, ev=None):
        x, out, ws = sets[i % len(sets)]
        hope_scan2d_forward(x, init, w.n_heads, 15, w.chunk, out, workspace=ws, stream=stream,
                            scan_events=ev, readout=args.readout, mem_chunk=args.mem_chunk, **vkw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    i = args.warmup
    while time.perf_counter() - t_warm < 0.2:  # clock settling, untimed
        step(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i, scan_ev[i])
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kernel_ms = [a.elapsed_time(b) for a, b in scan_ev]
    k_avg = float(np.mean(kernel_ms)) * 1e-3
    if args.copy_probe_mib > 0:  # a plain copy of known size for the HBM counter scale
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    tokens = w.scan_tokens(4)
    roof = roofline_numbers(w, readout=args.readout)
    kname = hope_scan2d_kernel_name(sets[0][0], w.n_heads, 15, w.chunk, readout=args.readout,
                                    mem_chunk=args.mem_chunk, **vkw)
    on_mfma = kname != "chain_kernel"
    achieved = roof["flops"] / k_avg
    # the fp32 VALU kernel runs every product in fp32 on the vector ALUs (157.3 TFLOP/s);
    # the MFMA kernels are held to the blend of the two classes' peaks
    t_roof = roof["t_compute"] if on_mfma else roof["flops"] / PEAK_FP32
    peak = roof["flops"] / t_roof
    k_med = float(np.median(kernel_ms)) * 1e-3
    rec = {
        "metric": METRIC,
        "value": tokens * args.steps / wall,
        "unit": "scan tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # inputs bf16, state and accumulation fp32; on the MFMA kernels the fp32 state's
        # products run as three bf16 products of a hi/lo split (about 2^-16 relative)
        "dtype": "bf16-in/f32-state(bf16x3)" if on_mfma else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "W": w.W, "D": w.D,
                   "n_heads": w.n_heads, "chunk": w.chunk or w.W, "dirs": 4, "x_dtype": w.dtype,
                   "state_dtype": "f32", "readout": args.readout, "variants": var,
                   "mem_chunk": args.mem_chunk},
        "roofline": {"bound": "mfma" if on_mfma else "alu", "achieved": achieved / 1e12,
                     "peak": peak / 1e12, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": recorded_traffic(w) if args.readout == "boundary" and not var else None,
                     "kernel": kname, "kernel_ms": k_avg * 1e3, "kernel_ms_median": k_med * 1e3,
                     "kernel_ms_p10_p90": [float(np.percentile(kernel_ms, 10)),
                                           float(np.percentile(kernel_ms, 90))],
                     "calls_timed": len(kernel_ms),
                     "t_roof_ms": t_roof * 1e3,
                     # the same flops at the bf16 matrix peak, counted as executed (hi/lo
                     # split products): the bound of this kernel's own instruction mix
                     "frac_as_executed": roof["t_as_executed"] / k_avg if on_mfma else None,
                     "call_ms": float(np.mean(call_ms)),
                     "call_ms_median": float(np.median(call_ms)),
                     "hbm_algorithmic_bytes": roof["hbm_bytes"],
                     "hbm_frac": roof["hbm_bytes"] / k_avg / PEAK_HBM},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp, readout=args.readout)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
