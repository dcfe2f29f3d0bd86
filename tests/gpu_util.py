"""Helpers for the GPU parity tests: inputs on the device, runs, comparisons.

Expected values always come from the oracle (``oracle`` package) on the same
seeded inputs; nothing here derives an expected value from the HIP library.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import pts_inputs as gen

DEV = "cuda:0"


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_device(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (any shape) -> contiguous bf16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def device_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def tol_for(out_dtype, k: int) -> float:
    """Max |D - ref| allowed for uniform[-1, 1] inputs: 2e-3 sqrt(K) for fp32 output,
    1e-2 sqrt(K) for bf16 output."""
    return (2e-3 if out_dtype == torch.float32 else 1e-2) * math.sqrt(max(k, 1))


def d_as_f64(d: torch.Tensor) -> np.ndarray:
    return d.detach().float().cpu().double().numpy() if d.dtype == torch.bfloat16 else \
        d.detach().cpu().double().numpy()


def check_exact(d: torch.Tensor, ref: np.ndarray, what: str) -> None:
    """Integer-valued inputs: fp32 output equals the exact sum; bf16 output equals
    the oracle's round-to-nearest-even of it, bit for bit."""
    if d.dtype == torch.float32:
        got = d.cpu().double().numpy()
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: {got[tuple(bad[0])]} != {ref[tuple(bad[0])]}"
    else:
        got = device_to_bits(d)
        want = oracle.bf16_round(ref)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{what}: {len(bad)} bf16 mismatches, first at {tuple(bad[0])}"


def check_close(d: torch.Tensor, ref: np.ndarray, k: int, what: str) -> float:
    got = d_as_f64(d)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    tol = tol_for(d.dtype, k)
    assert err <= tol, f"{what}: max |D - ref| = {err:.3g} > {tol:.3g}"
    return err


def check_counters(schedule, counters, tiles, workers):
    """Claim counters after a finished run: the live counters are back at zero.

    Single counter: every worker's loop ends on exactly one failed claim, so a
    run takes tiles + workers claims. Per-XCD counters: a request may also fail
    on several XCD ranges before it finds a tile, so at least that many.
    """
    assert counters[4] == 0, f"stage-flag waits ran out: {counters}"
    if schedule in ("static", "nonpersistent"):
        return
    assert counters[:2] == [0, 0], f"live counters not reset: {counters}"
    if schedule == "dynamic":
        assert counters[2] == tiles + workers, f"{counters[2]} claims, want {tiles + workers}"
    else:
        assert tiles + workers <= counters[2] <= tiles + 8 * (tiles + workers), counters


def run_single(m, n, k, a, b, out_dtype, schedule, tile=(0, 0), lda=0, ldb=0, ldd=0, num_workers=0, d=None,
               flags=0):
    """One plan, one run; D defaults to a NaN-filled (m x ldd) buffer. ld = 0 is packed."""
    import persistent_tile_scheduling_amd as pts
    if d is None:
        d = torch.full((max(m, 1), max(ldd or n, 1)), float("nan"), dtype=out_dtype, device=DEV)
    with pts.Plan([(m, n, k, lda, ldb, ldd)], out_dtype, tile, schedule, num_workers, flags) as p:
        p.run([(a, b, d)])
        torch.cuda.synchronize()
        counters = p.counters()
        info = (p.num_tiles, p.num_workers)
    return d, counters, info


def sample_entries(shapes, bm, bn, n_random, seed=0):
    """Per problem: the four corners of every output tile plus n_random uniform entries."""
    rng = np.random.default_rng(seed)
    out = []
    for (m, n) in shapes:
        rows, cols = [], []
        for r0 in range(0, m, bm):
            r1 = min(m, r0 + bm) - 1
            for c0 in range(0, n, bn):
                c1 = min(n, c0 + bn) - 1
                rows += [r0, r0, r1, r1]
                cols += [c0, c1, c0, c1]
        if m and n:
            rows += list(rng.integers(0, m, n_random))
            cols += list(rng.integers(0, n, n_random))
        out.append((np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)))
    return out


def oracle_sampled(seed, a_tid, b_tid, k, rows, cols):
    """Oracle values at (rows, cols) for A/B drawn from streams a_tid / b_tid
    (packed, uniform[-1,1]); only the needed rows of A and columns of B are
    regenerated on the host."""
    ur, rinv = np.unique(rows, return_inverse=True)
    uc, cinv = np.unique(cols, return_inverse=True)
    a_rows = np.concatenate([gen.uniform_bf16_bits(seed, a_tid, k, start=int(i) * k) for i in ur]) if k else \
        np.zeros(0, np.uint16)
    b_cols = np.concatenate([gen.uniform_bf16_bits(seed, b_tid, k, start=int(j) * k) for j in uc]) if k else \
        np.zeros(0, np.uint16)
    return oracle.gemm_entries(a_rows, b_cols, k, rinv, cinv)


def device_uniform(rows, cols, seed, tid) -> torch.Tensor:
    """(rows x cols) bf16 on the GPU, element (r, c) = stream index r * cols + c."""
    return gen.uniform_bf16_torch(rows * cols, seed, tid, DEV).view(rows, cols)


def check_sampled(d: torch.Tensor, rows, cols, ref: np.ndarray, k: int, what: str) -> float:
    got = d_as_f64(d[torch.as_tensor(rows, device=d.device), torch.as_tensor(cols, device=d.device)])
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    tol = tol_for(d.dtype, k)
    assert err <= tol, f"{what}: max |D - ref| = {err:.3g} > {tol:.3g} over {len(rows)} sampled entries"
    return err


def check_against_fp32_matmul(d: torch.Tensor, a: torch.Tensor, b: torch.Tensor, k: int, what: str,
                              row_block: int = 2048) -> float:
    """Full-size property check beside the oracle's sampled entries: every element
    against an fp32 product of the same bf16 values (torch, a library routine),
    within the same tolerance. Row blocks bound the temporary memory."""
    tol = tol_for(d.dtype, k)
    bf = b[:, :k].float()
    worst = 0.0
    for r0 in range(0, d.shape[0], row_block):
        r1 = min(d.shape[0], r0 + row_block)
        ref = a[r0:r1, :k].float() @ bf.t()
        err = (d[r0:r1, :ref.shape[1]].float() - ref).abs().max().item()
        worst = max(worst, err)
    assert worst <= tol, f"{what}: max |D - fp32 ref| = {worst:.3g} > {tol:.3g}"
    return worst


def band_rows(n, k, bm=256):
    """Tile rows per band of the plan's tile order: 8, or where B (n x k bf16)
    takes more than 128 MiB, the most tile rows (a multiple of 8 from 8 to 64)
    whose A rows (bm x k bf16 per tile row) fit in 192 MiB."""
    if n * k * 2 <= (128 << 20) or k == 0:
        return 8
    return min(64, max(8, (192 << 20) // (bm * k * 2) // 8 * 8))


def raster_tile(pos, tiles_m, tiles_n, band, rows=8, cols=4):
    """The plan's tile order inside one problem: bands of `band` tile rows,
    each walked in stripes of `cols` columns, each stripe in blocks of `rows`
    rows walked column by column: position -> (tile row, tile column)."""
    first = pos // (band * tiles_n) * band
    rows_in_band = min(band, tiles_m - first)
    in_band = pos - first * tiles_n
    stripe = in_band // (rows_in_band * cols)
    stripe_cols = min(cols, tiles_n - stripe * cols)
    in_stripe = in_band - stripe * rows_in_band * cols
    block = in_stripe // (rows * stripe_cols)
    block_rows = min(rows, rows_in_band - block * rows)
    in_block = in_stripe - block * rows * stripe_cols
    return first + block * rows + in_block % block_rows, stripe * cols + in_block // block_rows
