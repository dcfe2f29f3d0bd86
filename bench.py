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
concurrent 2^30-element int16 copy on a second stream limited to 64 compute
units; c6 64 grouped problems 1024 x 1024 with per-problem K_g in
{256..8192} (tiles of unequal cost), bf16 out.
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
    if name == "c6":
        ks = gen.grouped_k_draw(0)
        return dict(desc="grouped bf16 GEMM, 64 problems 1024x1024, K_g~U{256..8192}, bf16 out, one launch",
                    shapes=[(1024, 1024, k) for k in ks], out=torch.bfloat16, tile=(256, 256), copy=0)
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


class Concurrent:
    """The concurrent HBM-bound load of the copy workload: a grid-stride int16
    copy launched just before each GEMM run on a second stream. With
    copy_cus > 0 that stream is restricted to the first copy_cus compute
    units, so the copy holds part of the chip and the GEMM workers placed
    there start late."""

    def __init__(self, pts, n, copy_cus):
        import pts_inputs as gen
        import torch
        self.pts = pts
        self.n = n
        self.src = gen.uniform_bf16_torch(n, 0, gen.TENSOR_COPY_SRC, "cuda").view(torch.int16)
        self.dst = torch.empty_like(self.src)
        self.raw = pts.pts_stream_create_cu_masked(copy_cus) if copy_cus > 0 else None
        self.stream = self.raw if self.raw is not None else torch.cuda.Stream()
        self.blocks = 4 * copy_cus if copy_cus > 0 else 0

    def launch(self):
        self.pts.pts_copy_int16(self.src, self.dst, self.n, self.blocks, self.stream)

    def close(self):
        import torch
        torch.cuda.synchronize()
        if self.raw is not None:
            self.pts.pts_stream_destroy(self.raw)
            self.raw = None


def copy_alone_ms(conc, runs):
    """Median wall time of the concurrent copy by itself (synchronized per run)."""
    import torch
    ts = []
    for _ in range(runs + 2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        conc.launch()
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e3)
    ts = sorted(ts[2:])
    return ts[len(ts) // 2]


LATE = "+claim_after_tile"


def plan_args(pts, wl, key):
    """(schedule, flags) of a comparison key: a schedule name, or a name with
    the suffix '+claim_after_tile' (the same schedule with request-ahead off)."""
    if key.endswith(LATE):
        return key[:-len(LATE)], wl["flags"] | pts.GEMM_FLAG_CLAIM_AFTER_TILE
    return key, wl["flags"]


def claim_ahead_summary(results):
    """Kernel time with request-ahead off over the time with it on, per
    dynamic schedule (> 1: asking for the next tile early pays)."""
    out = {}
    for key, r in results.items():
        if key.endswith(LATE) and key[:-len(LATE)] in results and "kernel_ms_median" in r:
            out[key[:-len(LATE)]] = round(r["kernel_ms_median"] / results[key[:-len(LATE)]]["kernel_ms_median"], 4)
    return out


def time_headline(pts, wl, ops, schedule, steps, warmup, conc=None):
    """K timed steps of one schedule, wall clock plus per-launch HIP events."""
    import torch
    stream = torch.cuda.Stream()
    flops = sum(2.0 * m * n * k for (m, n, k) in wl["shapes"])
    sched, flags = plan_args(pts, wl, schedule)
    with pts.Plan(wl["shapes"], wl["out"], wl["tile"], sched, 0, flags) as plan:
        for _ in range(warmup):
            if conc is not None:
                conc.launch()
            plan.run(ops, stream)
        torch.cuda.synchronize()
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            if conc is not None:
                conc.launch()
            starts[i].record(stream)
            plan.run(ops, stream)
            ends[i].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        kms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
        info = dict(num_tiles=plan.num_tiles, num_workers=plan.num_workers, lds_bytes=plan.lds_bytes)
    avg = sum(kms) / len(kms)
    return dict(
        schedule=schedule,
        ms_per_step=wall * 1e3 / steps,
        tflops=flops * steps / wall / 1e12,
        kernel_ms_avg=avg,
        kernel_ms_median=sorted(kms)[len(kms) // 2],
        kernel_ms_min=min(kms),
        kernel_tflops=flops / (avg * 1e-3) / 1e12,
        **info,
    ), flops


def compare_schedules(pts, wl, ops, schedules, rounds, conc=None):
    """Every schedule run in turn, `rounds` times, the order rotated each round,
    so that clock and power drift fall on all schedules alike. Kernel times
    from HIP events on the launch stream; medians reported."""
    import torch
    stream = torch.cuda.Stream()
    flops = sum(2.0 * m * n * k for (m, n, k) in wl["shapes"])
    plans = {}
    for s in schedules:
        sched, flags = plan_args(pts, wl, s)
        plans[s] = pts.Plan(wl["shapes"], wl["out"], wl["tile"], sched, 0, flags)
    times = {s: [] for s in schedules}
    try:
        for s in schedules:
            if conc is not None:
                conc.launch()
            plans[s].run(ops, stream)
        torch.cuda.synchronize()
        for r in range(rounds):
            order = schedules[r % len(schedules):] + schedules[:r % len(schedules)]
            for s in order:
                if conc is not None:
                    conc.launch()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                plans[s].run(ops, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                times[s].append(e0.elapsed_time(e1))
    finally:
        for p in plans.values():
            p.close()
    out = {}
    for s, ts in times.items():
        med = sorted(ts)[len(ts) // 2]
        out[s] = dict(kernel_ms_median=med, kernel_ms_min=min(ts), kernel_tflops_median=flops / (med * 1e-3) / 1e12)
    return out


def tail_idle(pts, wl, ops, schedule, conc=None):
    """Fraction of worker-time idle after each worker's last tile, from the trace."""
    import torch
    stream = torch.cuda.Stream()
    sched, flags = plan_args(pts, wl, schedule)
    with pts.Plan(wl["shapes"], wl["out"], wl["tile"], sched, 0, flags) as plan:
        buf = torch.zeros(plan.trace_bytes() // 4 + 4, dtype=torch.int32, device="cuda")
        plan.set_trace(buf)
        for _ in range(2):
            if conc is not None:
                conc.launch()
            plan.run(ops, stream)
        torch.cuda.synchronize()
        tiles, workers = pts.decode_trace(buf, plan.num_tiles, plan.num_workers)
    start = workers["t_start"].astype("float64")
    end = workers["t_end"].astype("float64")
    span = end.max() - start.min()
    idle = float(((end.max() - end).sum()) / (len(end) * span)) if span > 0 else 0.0
    late = float(((start - start.min()).sum()) / (len(end) * span)) if span > 0 else 0.0
    per = workers["tiles"]
    busy_ns = (tiles["t_end"] - tiles["t_start"]).astype("float64").sum() * 10.0
    clock = float(tiles["cycles"].astype("float64").sum() / busy_ns) if busy_ns > 0 else None
    return dict(tail_idle_frac=idle, late_start_frac=late, span_us=span / 100.0,
                tiles_per_worker_min=int(per.min()), tiles_per_worker_max=int(per.max()),
                clock_ghz=clock)


def vendor_gemm(wl, ops, steps):
    """Context only: the vendor BLAS (torch.mm -> hipBLASLt) on the same single
    problem and operands, D = A . B with B given as its (n x k) transpose."""
    import torch
    (m, n, k), = wl["shapes"]
    a, b, _ = ops[0]
    out = torch.empty((m, n), dtype=wl["out"], device="cuda")
    if wl["out"] != torch.bfloat16:
        return None
    bt = b.t()
    for _ in range(5):
        torch.mm(a, bt, out=out)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        torch.mm(a, bt, out=out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    return dict(kernel_ms_avg=ms, tflops=2.0 * m * n * k / (ms * 1e-3) / 1e12, library="torch.mm (hipBLASLt)")


def kernel_source_digest(base=None) -> str:
    """sha256 over the HIP sources the GEMM kernel is built from, with comments
    and blank space removed (a comment edit does not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    base = base or os.path.join(ROOT, "persistent_tile_scheduling_amd", "csrc")
    for dirpath, _, files in sorted(os.walk(base)):
        for f in sorted(files):
            if f.endswith((".h", ".hip")):
                path = os.path.join(dirpath, f)
                text = open(path, encoding="utf-8").read()
                text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
                text = re.sub(r"//[^\n]*", " ", text)
                h.update(os.path.relpath(path, base).encode())
                h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload_name, schedule, wl):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload and schedule, or None when there is none or the kernel
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"gemm_{workload_name}_{schedule}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#")):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's name."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


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
                cpu_model=cpu_model(), logical_cpus=os.cpu_count(), seconds=t,
                sample=f"output rows 0..{rows - 1} (all {n} columns, K={k}) of problem 0, "
                       f"fp64 i-k-j loop (each element summed k ascending), OpenMP over rows")


IMBALANCED_SCHEDULES = ["static", "dynamic", "dynamic_xcd", "dynamic" + LATE, "dynamic_xcd" + LATE]


def imbalanced_comparison(pts, names, rounds, copy_cus):
    """The workloads where dynamic claiming should matter (ragged, grouped,
    concurrent copy): every schedule timed in interleaved rounds (medians of
    HIP-event kernel times), then one traced run each for the tail-idle and
    late-start fractions. Operands are freed before the next workload."""
    import torch
    out = {}
    for name in names:
        wl = workload(name)
        wl["tile"] = tuple(wl["tile"][:2])
        wl["flags"] = 0
        ops = make_operands(wl)
        conc = Concurrent(pts, wl["copy"], copy_cus) if wl["copy"] else None
        torch.cuda.synchronize()
        res = compare_schedules(pts, wl, ops, IMBALANCED_SCHEDULES, rounds, conc)
        for sched in IMBALANCED_SCHEDULES:
            res[sched].update(tail_idle(pts, wl, ops, sched, conc))
        if conc is not None:
            conc.close()
        base = res["static"]["kernel_ms_median"]
        entry = {
            "workload": wl["desc"],
            "tile": list(wl["tile"]),
            "copy_cus": copy_cus if wl["copy"] else None,
            "rounds": rounds,
            "schedules": {s: {k: (round(v, 5) if isinstance(v, float) else v) for k, v in r.items()}
                          for s, r in res.items()},
            "dynamic_vs_static": {s: round(base / r["kernel_ms_median"], 4)
                                  for s, r in res.items() if s != "static"},
            "claim_ahead": claim_ahead_summary(res),
        }
        out[name] = entry
        print(f"# imbalanced {name}: " + ", ".join(
            f"{s} {r['kernel_tflops_median']:.1f} TFLOP/s tail idle {r['tail_idle_frac']:.3f}"
            for s, r in res.items()) + f"; dynamic/static {entry['dynamic_vs_static']}; request-ahead off/on "
            f"{entry['claim_ahead']}", file=sys.stderr, flush=True)
        del ops, conc
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def tile_cycle_fit(pts, schedule="static", ks=(1024, 2048, 4096, 8192), mn=8192):
    """Shader cycles per tile against K (M = N = mn, bf16 out, 256x256 tiles):
    from the kernel's own trace, the median tile (start of the tile to the end
    of its epilogue) plus the median gap to the worker's next tile, fitted as
    boundary + per_k_tile * (K / 64). The boundary is what a tile costs beyond
    its k-tiles: decode, the first stage's load latency, the epilogue, the
    hand-over to the next tile."""
    import numpy as np
    import pts_inputs as gen
    import torch
    rows = []
    for k in ks:
        a = gen.uniform_bf16_torch(mn * k, 0, gen.TENSOR_A, "cuda").view(mn, k)
        b = gen.uniform_bf16_torch(mn * k, 0, gen.TENSOR_B, "cuda").view(mn, k)
        d = torch.empty((mn, mn), dtype=torch.bfloat16, device="cuda")
        with pts.Plan([(mn, mn, k)], torch.bfloat16, (256, 256), schedule) as p:
            buf = torch.zeros(p.trace_bytes() // 4 + 4, dtype=torch.int32, device="cuda")
            for _ in range(3):
                p.run([(a, b, d)])
            p.set_trace(buf)
            tile_cyc, gaps, clocks = [], [], []
            for _ in range(3):
                p.run([(a, b, d)])
                torch.cuda.synchronize()
                tiles, _ = pts.decode_trace(buf, p.num_tiles, p.num_workers)
                ns = (tiles["t_end"] - tiles["t_start"]).astype(np.float64) * 10.0
                clock = tiles["cycles"].astype(np.float64).sum() / ns.sum()
                order = np.lexsort((tiles["seq"], tiles["worker"]))
                ts = tiles["t_start"][order].astype(np.float64)
                te = tiles["t_end"][order].astype(np.float64)
                same = tiles["worker"][order][1:] == tiles["worker"][order][:-1]
                tile_cyc.append(float(np.median(tiles["cycles"].astype(np.float64))))
                gaps.append(float(np.median((ts[1:] - te[:-1])[same] * 10.0 * clock)) if same.any() else 0.0)
                clocks.append(clock)
        rows.append(dict(k=k, k_tiles=k // 64, tile_cycles=float(np.median(tile_cyc)), gap_cycles=float(np.median(gaps)),
                         clock_ghz=float(np.median(clocks))))
        print(f"# K={k}: median tile {rows[-1]['tile_cycles']:.0f} cycles, gap to the next tile "
              f"{rows[-1]['gap_cycles']:.0f}, clock {rows[-1]['clock_ghz']:.3f} GHz", file=sys.stderr, flush=True)
        del a, b, d
        torch.cuda.empty_cache()
    x = np.array([r["k_tiles"] for r in rows], dtype=np.float64)
    y = np.array([r["tile_cycles"] + r["gap_cycles"] for r in rows])
    (b0, b1), *_ = np.linalg.lstsq(np.vstack([np.ones_like(x), x]).T, y, rcond=None)
    return dict(schedule=schedule, mn=mn, rows=rows, boundary_cycles=float(b0), cycles_per_k_tile=float(b1),
                mfma_ideal_cycles_per_k_tile=2048)


def mfma_ceiling(pts, steps, warmup, isolated=15, ksteps=1024):
    """The matrix-unit ceiling probe (the default kernel's MFMA work with no
    memory traffic, one workgroup of 8 waves per compute unit; ksteps = 1024
    is the FLOP of one 8192^3 GEMM): `steps` launches back to back after
    `warmup`, as the headline times the GEMM, then `isolated` single launches
    with idle time between them. Operand fragments are drawn like A and B."""
    import numpy as np
    import pts_inputs as gen
    import torch
    frags = gen.uniform_bf16_torch(pts.PTS_MFMA_CEILING_FRAG_BYTES // 2, 0, gen.TENSOR_A, "cuda")
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stamps = torch.zeros(blocks * 2, dtype=torch.int64, device="cuda")
    flops = blocks * 8 * ksteps * 32 * 16384.0
    stream = torch.cuda.Stream()

    def clock_ghz():
        st = stamps.view(-1, 2).cpu().numpy().astype(np.float64)
        return float(np.median(st[:, 0] / (st[:, 1] * 10.0)))

    for _ in range(warmup):
        pts.pts_mfma_ceiling(frags, out, stamps, blocks, ksteps, stream)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        pts.pts_mfma_ceiling(frags, out, stamps, blocks, ksteps, stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    back_clock = clock_ghz()
    iso, iso_clock = [], []
    for _ in range(isolated):
        time.sleep(0.05)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pts.pts_mfma_ceiling(frags, out, stamps, blocks, ksteps, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        iso.append(e0.elapsed_time(e1))
        iso_clock.append(clock_ghz())
    avg = sum(kms) / len(kms)
    med_iso = sorted(iso)[len(iso) // 2]
    return dict(blocks=blocks, waves_per_block=8, k_steps=ksteps, flop_per_launch=flops,
                back_to_back=dict(launches=steps, kernel_ms_avg=round(avg, 5),
                                  tflops=round(flops / (avg * 1e-3) / 1e12, 1),
                                  frac=round(flops / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  clock_ghz_last_launch=round(back_clock, 3)),
                isolated=dict(launches=isolated, kernel_ms_median=round(med_iso, 5),
                              tflops=round(flops / (med_iso * 1e-3) / 1e12, 1),
                              frac=round(flops / (med_iso * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              clock_ghz_median=round(float(np.median(iso_clock)), 3)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--schedules", default="static,dynamic,dynamic_xcd,nonpersistent,dynamic_xcd" + LATE,
                    help="comma list; a '+claim_after_tile' suffix turns the dynamic schedules' request-ahead off")
    ap.add_argument("--tile-k", type=int, default=0, help="k-tile depth (0 = library default)")
    ap.add_argument("--stages", type=int, default=0, help="LDS ring stages (0 = library default)")
    ap.add_argument("--load-path", type=int, default=0, help="1 = global->LDS, 2 = via registers (0 = default)")
    ap.add_argument("--waves", type=int, default=0, help="waves per workgroup, 4 or 8 (0 = default)")
    ap.add_argument("--mfma", type=int, default=0, help="MFMA block edge, 16 or 32 (0 = default)")
    ap.add_argument("--problem-order", default="deepest_first", choices=["deepest_first", "as_given"],
                    help="tile order of grouped problems: deepest first (default) or as given")
    ap.add_argument("--stage-sync", default="barrier", choices=["barrier", "fused", "merged"],
                    help="stage hand-off: workgroup barrier, or LDS full/empty counters (2 or 3 words per stage)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--compare-rounds", type=int, default=10,
                    help="interleaved rounds of every schedule for the comparison (0 = skip)")
    ap.add_argument("--no-vendor", dest="vendor", action="store_false",
                    help="skip the vendor BLAS context timing")
    ap.add_argument("--vendor-only", action="store_true",
                    help="time only the vendor BLAS on the workload's operands (for side-by-side profiles)")
    ap.add_argument("--copy-cus", type=int, default=64,
                    help="compute units the concurrent copy may use (0 = all, unmasked stream)")
    ap.add_argument("--imbalanced", default="c3,c4,c5",
                    help="with the 8192^3 headline: also compare the schedules on these workloads ('' = skip)")
    ap.add_argument("--imbalanced-rounds", type=int, default=7,
                    help="interleaved rounds per schedule on each imbalanced workload")
    ap.add_argument("--tile-cycles", action="store_true",
                    help="only fit shader cycles per tile against K (8192 x 8192 x K, K = 1024..8192) and print it")
    ap.add_argument("--no-ceiling", dest="ceiling", action="store_false",
                    help="leave the matrix-unit ceiling probe out of the default 8192^3 line")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the matrix-unit ceiling probe (the GEMM's MFMA work without memory traffic)")
    ap.add_argument("--calibration-copy", type=int, default=0,
                    help="also run one int16 copy of this many elements (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run the same kernel on its own row block of tiles).", file=sys.stderr)
        sys.exit(2)

    import torch
    import persistent_tile_scheduling_amd as pts

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.tile_cycles:
        fit = tile_cycle_fit(pts)
        print(json.dumps({"tile_cycle_fit": fit}), flush=True)
        return
    if args.mfma_ceiling:
        ceil = mfma_ceiling(pts, args.steps, args.warmup)
        print(f"# MFMA ceiling: back to back {ceil['back_to_back']['tflops']} TFLOP/s "
              f"(frac {ceil['back_to_back']['frac']}), isolated {ceil['isolated']['tflops']} TFLOP/s",
              file=sys.stderr, flush=True)
        print(json.dumps({"mfma_ceiling": ceil}), flush=True)
        return
    wl = workload(args.workload)
    wl["tile"] = tuple(wl["tile"][:2]) + (args.tile_k, args.stages, args.load_path, args.waves, args.mfma)
    wl["flags"] = {"barrier": 0, "fused": pts.GEMM_FLAG_STAGE_FLAGS_FUSED,
                   "merged": pts.GEMM_FLAG_STAGE_FLAGS_MERGED}[args.stage_sync]
    if args.problem_order == "as_given":
        wl["flags"] |= pts.GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN
    print(f"# workload {args.workload}: {wl['desc']}", file=sys.stderr, flush=True)
    ops = make_operands(wl)
    if args.vendor_only:
        vendor = vendor_gemm(wl, ops, args.steps) if len(wl["shapes"]) == 1 else None
        if vendor is None:
            print("--vendor-only needs a single-problem workload with bf16 output", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"vendor_library": vendor, "config": {"workload": wl["desc"]}}), flush=True)
        return
    conc = Concurrent(pts, wl["copy"], args.copy_cus) if wl["copy"] else None
    torch.cuda.synchronize()

    if args.calibration_copy:
        n = args.calibration_copy
        src = torch.zeros(n, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        pts.pts_copy_int16(src, dst, n)
        torch.cuda.synchronize()
        del src, dst

    schedules = args.schedules.split(",")
    head_sched = "dynamic_xcd" if "dynamic_xcd" in schedules else schedules[-1]
    head, flops = time_headline(pts, wl, ops, head_sched, args.steps, args.warmup, conc)
    print(f"# headline {head_sched}: {head['tflops']:.1f} TFLOP/s wall, {head['kernel_tflops']:.1f} TFLOP/s "
          f"kernel ({head['kernel_ms_avg']:.4f} ms avg), {100 * head['kernel_tflops'] / PEAK_BF16_TFLOPS:.1f}% "
          f"of peak", file=sys.stderr, flush=True)
    results = {}
    if len(schedules) > 1 and args.compare_rounds > 0:
        results = compare_schedules(pts, wl, ops, schedules, args.compare_rounds, conc)
        for sched, r in results.items():
            print(f"# compare {sched}: median {r['kernel_ms_median']:.4f} ms, {r['kernel_tflops_median']:.1f} "
                  f"TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_trace:
        for sched in schedules:
            r = results.setdefault(sched, {})
            r.update(tail_idle(pts, wl, ops, sched, conc))
            print(f"# trace {sched}: tail idle {r['tail_idle_frac']:.3f}, late start {r['late_start_frac']:.3f}",
                  file=sys.stderr, flush=True)
    without_copy, copy_alone = None, None
    if conc is not None:
        if len(schedules) > 1 and args.compare_rounds > 0:
            # the same comparison with nothing else on the chip, and the copy on its own
            without_copy = compare_schedules(pts, wl, ops, schedules, args.compare_rounds)
            for sched, r in without_copy.items():
                print(f"# without copy {sched}: median {r['kernel_ms_median']:.4f} ms, "
                      f"{r['kernel_tflops_median']:.1f} TFLOP/s", file=sys.stderr, flush=True)
            copy_alone = copy_alone_ms(conc, 10)
            print(f"# copy alone on {args.copy_cus} CUs: {copy_alone:.4f} ms", file=sys.stderr, flush=True)
        conc.close()
    vendor = vendor_gemm(wl, ops, args.steps) if args.vendor and len(wl["shapes"]) == 1 else None
    if vendor:
        print(f"# vendor {vendor['library']}: {vendor['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    ceiling = None
    if args.ceiling and args.workload == "c2":
        # the same launch count back to back, the GEMM's MFMA work alone
        ceiling = mfma_ceiling(pts, args.steps, args.warmup)
        print(f"# MFMA ceiling: back to back {ceiling['back_to_back']['tflops']} TFLOP/s", file=sys.stderr,
              flush=True)

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
        "config": {"workload": wl["desc"], "schedule": head_sched,
                   "shapes": wl["shapes"] if len(wl["shapes"]) <= 4 else f"{len(wl['shapes'])} problems",
                   "tile": list(wl["tile"]), "out_dtype": str(wl["out"]).replace("torch.", ""),
                   "copy_cus": args.copy_cus if wl["copy"] else None, "stage_sync": args.stage_sync,
                   "problem_order": args.problem_order},
        "roofline": {"bound": "mfma", "achieved": round(head["kernel_tflops"], 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(head["kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload, head_sched, wl) if args.stage_sync == "barrier" else None,
                     "kernel": "pts::gemm_persistent_kernel", "flop_per_launch": flops,
                     "kernel_ms_avg": round(head["kernel_ms_avg"], 5)},
        "schedules": {k: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                      for k, v in results.items()},
    }
    clock = results.get(head_sched, {}).get("clock_ghz")
    if clock:
        # the same launch against the MFMA peak at the clock the chip actually held
        peak_at_clock = 256 * 4096 * clock * 1e9 / 1e12
        line["roofline"]["clock_ghz_measured"] = round(clock, 3)
        line["roofline"]["peak_at_measured_clock"] = round(peak_at_clock, 1)
        line["roofline"]["frac_at_measured_clock"] = round(head["kernel_tflops"] / peak_at_clock, 4)
    if vendor:
        line["vendor_library"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in vendor.items()}
    if ceiling:
        b2b = ceiling["back_to_back"]
        line["mfma_ceiling"] = {"kernel": "pts::mfma_ceiling_kernel", "tflops": b2b["tflops"], "frac": b2b["frac"],
                                "clock_ghz": b2b["clock_ghz_last_launch"],
                                "gemm_over_ceiling": round(head["kernel_tflops"] / b2b["tflops"], 4)}
    if "static" in results and "kernel_ms_median" in results["static"]:
        line["dynamic_vs_static"] = {s: round(results["static"]["kernel_ms_median"] / r["kernel_ms_median"], 4)
                                     for s, r in results.items() if s != "static" and "kernel_ms_median" in r}
    if claim_ahead_summary(results):
        line["claim_ahead"] = claim_ahead_summary(results)
    if without_copy:
        line["without_copy"] = {s: {"kernel_ms_median": round(r["kernel_ms_median"], 5),
                                    "kernel_tflops_median": round(r["kernel_tflops_median"], 2)}
                                for s, r in without_copy.items()}
        line["copy_alone_ms"] = round(copy_alone, 5)
    if args.workload == "c2" and args.imbalanced and args.stage_sync == "barrier" and not any(
            (args.tile_k, args.stages, args.load_path, args.waves, args.mfma)):
        del ops
        torch.cuda.empty_cache()
        line["imbalanced"] = imbalanced_comparison(pts, args.imbalanced.split(","), args.imbalanced_rounds,
                                                   args.copy_cus)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
