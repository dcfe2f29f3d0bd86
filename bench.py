#!/usr/bin/env python3
"""Benchmark: bf16 GEMM TFLOP/s and % of MI355X dense bf16 MFMA peak, static vs
dynamic tile schedule, one GPU.

A step is one gemm_run of the whole workload (one persistent launch) with the
inputs already resident in HBM. Every schedule named by --schedules is timed
(static grid-stride, dynamic single-counter claiming, dynamic per-XCD
claiming); the JSON line's `value` is the per-XCD dynamic schedule's
whole-job throughput (else the single-counter one's) and the others are
reported beside it. Kernel durations come from HIP events recorded on the
stream the kernel is launched on.

Workloads (--workload): c2 (default) 8192^3 bf16 out 256x256 tiles; c1 256^3
fp32 out 64x64 tiles; c3 5000x7000x3000 fp32 out; c4 64 grouped problems
M_g in {128..4096}, N = K = 4096, bf16 out; c5 16384^2 x 8192 bf16 out beside a
concurrent 2^30-element int16 copy on a second stream.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # 256 CUs x 4096 dense bf16 FLOP/clk x 2.4 GHz
METRIC = "bf16 GEMM TFLOP/s and % MFMA peak, dynamic vs static tile schedule"


def workload(name: str):
    import pts_inputs as gen
    import torch
    if name == "c1":
        return dict(desc="bf16 GEMM 256x256x256, fp32 out, 64x64 tiles", shapes=[(256, 256, 256)],
                    out=torch.float32, tile=(64, 64), copy=0)
    if name == "c2":
        return dict(desc="bf16 GEMM 8192x8192x8192, A row-major, B column-major, bf16 out, 256x256 tiles",
                    shapes=[(8192, 8192, 8192)], out=torch.bfloat16, tile=(256, 256), copy=0)
    if name == "c3":
        return dict(desc="ragged bf16 GEMM 5000x7000x3000, fp32 out, 256x256 tiles",
                    shapes=[(5000, 7000, 3000)], out=torch.float32, tile=(256, 256), copy=0)
    if name == "c4":
        ms = gen.grouped_m_draw(0)
        return dict(desc="grouped bf16 GEMM, 64 problems M_g~U{128..4096}, N=K=4096, bf16 out, one launch",
                    shapes=[(m, 4096, 4096) for m in ms], out=torch.bfloat16, tile=(256, 256), copy=0)
    if name == "c5":
        return dict(desc="bf16 GEMM 16384x16384x8192, bf16 out, beside a concurrent 2^30 int16 copy",
                    shapes=[(16384, 16384, 8192)], out=torch.bfloat16, tile=(256, 256), copy=1 << 30)
    raise SystemExit(f"unknown workload {name}")


def make_operands(wl, seed=0):
    import pts_inputs as gen
    import torch
    ops = []
    grouped = len(wl["shapes"]) > 1
    for g, (m, n, k) in enumerate(wl["shapes"]):
        ta, tb = gen.group_tensor_ids(g) if grouped else (gen.TENSOR_A, gen.TENSOR_B)
        a = gen.uniform_bf16_torch(m * k, seed, ta, "cuda").view(m, k)
        b = gen.uniform_bf16_torch(n * k, seed, tb, "cuda").view(n, k)
        d = torch.empty((m, n), dtype=wl["out"], device="cuda")
        ops.append((a, b, d))
    return ops


def time_schedule(pts, wl, ops, schedule, steps, warmup, copy_bufs=None):
    import torch
    stream = torch.cuda.Stream()
    copy_stream = torch.cuda.Stream() if copy_bufs is not None else None
    flops = sum(2.0 * m * n * k for (m, n, k) in wl["shapes"])
    with pts.Plan(wl["shapes"], wl["out"], wl["tile"], schedule) as plan:
        def one():
            if copy_bufs is not None:
                pts.pts_copy_int16(copy_bufs[0], copy_bufs[1], copy_bufs[0].numel(), 0, copy_stream)
            plan.run(ops, stream)
        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            if copy_bufs is not None:
                pts.pts_copy_int16(copy_bufs[0], copy_bufs[1], copy_bufs[0].numel(), 0, copy_stream)
            starts[i].record(stream)
            plan.run(ops, stream)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        info = dict(num_tiles=plan.num_tiles, num_workers=plan.num_workers, lds_bytes=plan.lds_bytes)
    kms_sorted = sorted(kms)
    avg = sum(kms) / len(kms)
    return dict(
        schedule=schedule,
        ms_per_step=wall * 1e3 / steps,
        tflops=flops * steps / wall / 1e12,
        kernel_ms_avg=avg,
        kernel_ms_median=kms_sorted[len(kms) // 2],
        kernel_ms_min=kms_sorted[0],
        kernel_tflops=flops / (avg * 1e-3) / 1e12,
        frac_of_peak=flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        **info,
    ), flops


def tail_idle(pts, wl, ops, schedule, copy_bufs=None):
    """Fraction of worker-time idle after each worker's last tile, from the trace."""
    import torch
    stream = torch.cuda.Stream()
    copy_stream = torch.cuda.Stream() if copy_bufs is not None else None
    with pts.Plan(wl["shapes"], wl["out"], wl["tile"], schedule) as plan:
        buf = torch.zeros(plan.trace_bytes() // 4 + 4, dtype=torch.int32, device="cuda")
        plan.set_trace(buf)
        for _ in range(2):
            if copy_bufs is not None:
                pts.pts_copy_int16(copy_bufs[0], copy_bufs[1], copy_bufs[0].numel(), 0, copy_stream)
            plan.run(ops, stream)
        torch.cuda.synchronize()
        tiles, workers = pts.decode_trace(buf, plan.num_tiles, plan.num_workers)
    start = workers["t_start"].astype("float64")
    end = workers["t_end"].astype("float64")
    span = end.max() - start.min()
    idle = float(((end.max() - end).sum()) / (len(end) * span)) if span > 0 else 0.0
    late = float(((start - start.min()).sum()) / (len(end) * span)) if span > 0 else 0.0
    per = workers["tiles"]
    return dict(tail_idle_frac=idle, late_start_frac=late, span_us=span / 100.0,
                tiles_per_worker_min=int(per.min()), tiles_per_worker_max=int(per.max()))


def cpu_baseline(wl, budget_s: float):
    """The oracle on a bounded row sample of the workload's first problem."""
    import numpy as np
    import oracle
    import pts_inputs as gen
    m, n, k = wl["shapes"][0]
    grouped = len(wl["shapes"]) > 1
    ta, tb = gen.group_tensor_ids(0) if grouped else (gen.TENSOR_A, gen.TENSOR_B)
    b = gen.uniform_bf16_bits(0, tb, n * k)
    rows = 1
    t = 0.0
    while True:
        a = gen.uniform_bf16_bits(0, ta, rows * k)
        t0 = time.perf_counter()
        oracle.gemm(a, b, rows, n, k)
        t = time.perf_counter() - t0
        if t >= budget_s * 0.5 or rows >= m:
            break
        rows = min(m, max(rows * 2, int(rows * budget_s / max(t, 1e-3))))
    flops = 2.0 * rows * n * k
    return dict(value=flops / t / 1e12, unit="TFLOP/s", cores=oracle.max_threads(), kind="oracle",
                seconds=t, sample=f"output rows 0..{rows - 1} (all {n} columns, K={k}) of problem 0, "
                                  f"fp64 triple loop, OpenMP over rows")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--schedules", default="static,dynamic,dynamic_xcd")
    ap.add_argument("--tile-k", type=int, default=0, help="k-tile depth (0 = library default)")
    ap.add_argument("--stages", type=int, default=0, help="LDS ring stages (0 = library default)")
    ap.add_argument("--load-path", type=int, default=0, help="1 = global->LDS, 2 = via registers (0 = default)")
    ap.add_argument("--waves", type=int, default=0, help="waves per workgroup, 4 or 8 (0 = default)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--calibration-copy", type=int, default=0,
                    help="also run one int16 copy of this many elements (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each GPU would run the same kernel on its own row block of tiles).", file=sys.stderr)
        sys.exit(2)

    import torch
    import persistent_tile_scheduling_amd as pts

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    wl = workload(args.workload)
    wl["tile"] = tuple(wl["tile"][:2]) + (args.tile_k, args.stages, args.load_path, args.waves)
    print(f"# workload {args.workload}: {wl['desc']}", file=sys.stderr, flush=True)
    ops = make_operands(wl)
    copy_bufs = None
    if wl["copy"]:
        import pts_inputs as gen
        src = gen.uniform_bf16_torch(wl["copy"], 0, gen.TENSOR_COPY_SRC, "cuda").view(torch.int16)
        copy_bufs = (src, torch.empty_like(src))
    torch.cuda.synchronize()

    if args.calibration_copy:
        n = args.calibration_copy
        src = torch.zeros(n, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        pts.pts_copy_int16(src, dst, n)
        torch.cuda.synchronize()
        del src, dst

    results = {}
    flops = None
    for sched in args.schedules.split(","):
        r, flops = time_schedule(pts, wl, ops, sched, args.steps, args.warmup, copy_bufs)
        print(f"# {sched}: {r['kernel_tflops']:.1f} TFLOP/s kernel, {r['tflops']:.1f} TFLOP/s wall, "
              f"{r['kernel_ms_avg']:.4f} ms avg kernel, {100 * r['frac_of_peak']:.1f}% of peak",
              file=sys.stderr, flush=True)
        if not args.no_trace:
            r.update(tail_idle(pts, wl, ops, sched, copy_bufs))
        results[sched] = r

    head = results.get("dynamic_xcd") or results.get("dynamic") or next(iter(results.values()))
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["desc"], "schedule": head["schedule"],
                   "shapes": wl["shapes"] if len(wl["shapes"]) <= 4 else f"{len(wl['shapes'])} problems",
                   "tile": list(wl["tile"]), "out_dtype": str(wl["out"]).replace("torch.", "")},
        "roofline": {"bound": "mfma", "achieved": round(head["kernel_tflops"], 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(head["kernel_tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "pts::gemm_persistent_kernel", "flop_per_launch": flops},
        "schedules": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in results.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
