"""GPU tests of the persistent tile scheduler (bit-exact index work).

* The scheduler probe replays the example of "Advanced scheduling: Cluster
  Launch Control", section "Limits of the static persistent scheduler":
  12 tiles, 4 workers. Static grid-stride must reproduce the printed table
  (tests/golden), also when worker 3 starts only after the others finished
  (the launch tail: it still owns 3, 7, 11). Dynamic claiming must process
  every tile exactly once and leave nothing for the late worker.
* Per-XCD claiming (one counter per XCD over a contiguous range of tile
  positions, stealing from the other ranges once the own one is used up) must
  also hand out every position exactly once; a worker only moves on to a
  range farther from its own XCD, and inside a range its claims increase.
* The GEMM kernel's own per-tile trace must cover every output tile of the
  problem exactly once, follow the static assignment in static mode, and end
  each dynamic run with the claim counters reset.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import pts_inputs as gen
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _golden(golden_dir):
    table = {}
    for line in open(os.path.join(golden_dir, "static_grid_stride_12_tiles_4_workers.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            w, ts = line.split(":")
            table[int(w)] = [int(t) for t in ts.split()]
    return table


def _probe(pts, tiles, workers, schedule, gate=-1, work_ns=20000, maxpw=None, counters=None):
    maxpw = maxpw or max(tiles, 1)
    out = torch.full((workers, maxpw), -1, dtype=torch.int32, device=U.DEV)
    counts = torch.full((workers,), -1, dtype=torch.int32, device=U.DEV)
    if counters is None:
        counters = torch.zeros(pts.GEMM_SCHED_COUNTER_BYTES // 4, dtype=torch.int32, device=U.DEV)
    status = torch.zeros(1, dtype=torch.int32, device=U.DEV)
    pts.pts_sched_probe(tiles, workers, schedule, gate, work_ns, 2_000_000, out, counts, maxpw, counters, status)
    torch.cuda.synchronize()
    assert status.item() == 0, "gate wait expired"
    cnt = counts.cpu().tolist()
    rows = out.cpu().tolist()
    per_worker = [rows[w][:cnt[w]] for w in range(workers)]
    return per_worker, _counter_summary(counters)


def _counter_summary(counters):
    """[claim, exit, final claim total, runs] followed by the 8 per-XCD counters."""
    c = counters.cpu().tolist()
    return [c[0], c[32], c[64], c[65]] + [c[1024 * (x + 1)] for x in range(8)]


def test_probe_static_matches_printed_example(pts, golden_dir):
    per_worker, _ = _probe(pts, 12, 4, pts.GEMM_SCHEDULE_STATIC)
    assert {w: ts for w, ts in enumerate(per_worker)} == _golden(golden_dir)


def test_probe_static_late_worker_keeps_its_tiles(pts, golden_dir):
    per_worker, _ = _probe(pts, 12, 4, pts.GEMM_SCHEDULE_STATIC, gate=3)
    assert per_worker[3] == [3, 7, 11]
    assert {w: ts for w, ts in enumerate(per_worker)} == _golden(golden_dir)


def test_probe_dynamic_exactly_once(pts):
    per_worker, counters = _probe(pts, 12, 4, pts.GEMM_SCHEDULE_DYNAMIC)
    oracle.check_dynamic_claims(per_worker, 12)
    # every worker's loop ended on exactly one failed claim: 12 + 4 claims
    assert counters[:4] == [0, 0, 16, 1]


def test_probe_dynamic_late_worker_finds_nothing(pts):
    per_worker, counters = _probe(pts, 12, 4, pts.GEMM_SCHEDULE_DYNAMIC, gate=3)
    oracle.check_dynamic_claims(per_worker, 12)
    assert per_worker[3] == []
    assert counters[2] == 16


def test_probe_dynamic_at_scale_and_repeated(pts):
    # one counter block across runs: each run must leave it reset for the next
    shared = torch.zeros(pts.GEMM_SCHED_COUNTER_BYTES // 4, dtype=torch.int32, device=U.DEV)
    for run in range(3):
        per_worker, counters = _probe(pts, 4096, 256, pts.GEMM_SCHEDULE_DYNAMIC, work_ns=2000, counters=shared)
        oracle.check_dynamic_claims(per_worker, 4096)
        assert counters[:4] == [0, 0, 4096 + 256, run + 1]


def test_probe_static_at_scale(pts):
    per_worker, _ = _probe(pts, 1000, 256, pts.GEMM_SCHEDULE_STATIC, work_ns=1000)
    assert per_worker == oracle.static_assignment(1000, 256)


def _part_begin(n, parts, p):
    q, rem = divmod(n, parts)
    return p * q + min(p, rem)


def static_position(t, num_tiles, round_size):
    """Position of logical index t: each round of round_size logical indices is
    dealt so that the indices = x (mod 8) -- one XCD's workers -- get one
    contiguous run of positions."""
    base = (t // round_size) * round_size
    r = min(round_size, num_tiles - base)
    u = t - base
    return base + _part_begin(r, 8, u % 8) + u // 8


def check_xcd_claims(claims, worker_xcd, num_tiles, num_workers):
    """Per-XCD claiming: `claims` per worker are XCD * 2^24 + counter value v,
    meaning logical index XCD + 8 v at its static position."""
    positions = []
    for w, seq in enumerate(claims):
        dists, last = [], {}
        for c in seq:
            x, v = c >> 24, c & 0xFFFFFF
            t = x + 8 * v
            assert 0 <= x < 8 and t < num_tiles, f"worker {w}: claim {c} outside XCD {x}'s sequence"
            positions.append(static_position(t, num_tiles, num_workers))
            assert v > last.get(x, -1), f"worker {w}: claims in XCD {x}'s sequence not increasing"
            last[x] = v
            dists.append((x - worker_xcd[w]) % 8)
        assert dists == sorted(dists), f"worker {w} went back to a nearer XCD: {dists}"
    assert sorted(positions) == list(range(num_tiles)), "positions not covered exactly once"
    return positions


def test_probe_dynamic_xcd_exactly_once(pts):
    for tiles, workers, work in ((12, 4, 20000), (4096, 256, 2000), (1000, 256, 500), (7, 9, 1000)):
        per_worker, counters = _probe(pts, tiles, workers, pts.GEMM_SCHEDULE_DYNAMIC_XCD, work_ns=work)
        assert sorted(t for ts in per_worker for t in ts) == list(range(tiles))
        assert counters[:2] == [0, 0] and counters[4:12] == [0] * 8
        assert counters[2] >= tiles + workers


def test_probe_dynamic_xcd_late_worker_finds_nothing(pts):
    per_worker, counters = _probe(pts, 12, 4, pts.GEMM_SCHEDULE_DYNAMIC_XCD, gate=3)
    assert sorted(t for ts in per_worker for t in ts) == list(range(12))
    assert per_worker[3] == []


def _traced_run(pts, shapes, schedule, tile=(0, 0), num_workers=0, out_dtype=torch.float32, k=64, flags=0):
    tensors = []
    for (m, n) in shapes:
        tensors.append((torch.zeros((max(m, 1), k), dtype=torch.bfloat16, device=U.DEV),
                        torch.zeros((max(n, 1), k), dtype=torch.bfloat16, device=U.DEV),
                        torch.empty((max(m, 1), max(n, 1)), dtype=out_dtype, device=U.DEV)))
    with pts.Plan([(m, n, k) for (m, n) in shapes], out_dtype, tile, schedule, num_workers, flags) as p:
        buf = torch.zeros(p.trace_bytes() // 4 + 4, dtype=torch.int32, device=U.DEV)
        p.set_trace(buf)
        p.run(tensors)
        torch.cuda.synchronize()
        tiles, workers = pts.decode_trace(buf, p.num_tiles, p.num_workers)
        return tiles.copy(), workers.copy(), p.num_tiles, p.num_workers, p.counters()


@pytest.mark.parametrize("m,n,k", [(13000, 8200, 8200), (5000, 7000, 64)])
def test_tile_order_bands(pts, m, n, k):
    """The kernel's position -> tile map, read from its trace, is the banded
    order: wide bands where B (n x k bf16) exceeds 128 MiB (here 40 rows, with
    a partial last band, a partial last block and a ragged last stripe), 8-row
    bands otherwise."""
    U.log(f"tile order: {m} x {n} x {k}, band {U.band_rows(n, k)}")
    tiles, _, nt, _, _ = _traced_run(pts, [(m, n)], "static", (256, 256), k=k)
    tiles_m, tiles_n = -(-m // 256), -(-n // 256)
    assert nt == tiles_m * tiles_n
    band = U.band_rows(n, k)
    for pos, r0, c0 in zip(tiles["tile"].tolist(), tiles["row0"].tolist(), tiles["col0"].tolist()):
        assert (r0 // 256, c0 // 256) == U.raster_tile(pos, tiles_m, tiles_n, band), f"position {pos}"


@pytest.mark.parametrize("schedule", ["static", "dynamic", "dynamic_xcd", "nonpersistent"])
@pytest.mark.parametrize("shapes,tile", [([(5000, 7000)], (256, 256)), ([(256, 256)], (64, 64)),
                                         ([(300, 200), (0, 10), (1000, 64), (1, 1)], (128, 128)),
                                         ([(20000, 2048)], (256, 256))])
def test_gemm_trace_covers_every_tile_once(pts, schedule, shapes, tile):
    tiles, workers, nt, nw, counters = _traced_run(pts, shapes, schedule, tile)
    # every output tile of every problem exactly once ...
    want = sorted((g, r0, c0) for (g, r0, c0, _, _) in oracle.tile_coords(shapes, *tile))
    got = sorted(zip(tiles["group"].tolist(), tiles["row0"].tolist(), tiles["col0"].tolist()))
    assert got == want
    # ... and every tile position exactly once
    assert sorted(tiles["tile"].tolist()) == list(range(nt))
    order = np.lexsort((tiles["seq"], tiles["worker"]))
    per_worker = [[] for _ in range(nw)]
    for i in order:
        per_worker[tiles["worker"][i]].append(int(tiles["claim"][i]))
    assert [len(p) for p in per_worker] == workers["tiles"].tolist()
    for w, p in enumerate(per_worker):
        seqs = sorted(int(x) for x in tiles["seq"][tiles["worker"] == w])
        assert seqs == list(range(len(p)))
    assert workers["worker"].tolist() == list(range(nw))
    assert np.all(tiles["t_end"] >= tiles["t_start"])
    span_ns = (tiles["t_end"] - tiles["t_start"]).astype(np.float64).sum() * 10.0
    if span_ns > 0:
        clock = tiles["cycles"].astype(np.float64).sum() / span_ns
        assert 0.3 < clock < 3.0, f"implausible shader clock {clock:.3f} GHz"
    assert np.all(tiles["xcc_id"] == workers["xcc_id"][tiles["worker"]])
    if schedule == "static":
        assert per_worker == oracle.static_assignment(nt, nw)
        assert all(int(p) == static_position(int(c), nt, nw) for p, c in zip(tiles["tile"], tiles["claim"]))
    elif schedule == "nonpersistent":
        assert nw == nt and per_worker == [[w] for w in range(nw)]
    elif schedule == "dynamic":
        assert np.array_equal(tiles["claim"], tiles["tile"])
        oracle.check_dynamic_claims(per_worker, nt)
    else:
        positions = check_xcd_claims(per_worker, (workers["xcc_id"] % 8).tolist(), nt, nw)
        flat = [tiles["tile"][i] for i in order]
        assert positions == [int(t) for t in flat]
    U.check_counters(schedule, counters, nt, nw)


def test_copy_kernel(pts):
    for n in (1, 7, 8, 9, 4096 + 3, (1 << 22) + 5):
        src = torch.randint(-32768, 32767, (n,), dtype=torch.int16, device=U.DEV)
        dst = torch.full((n + 40,), 1234, dtype=torch.int16, device=U.DEV)
        pts.pts_copy_int16(src, dst, n)
        torch.cuda.synchronize()
        assert torch.equal(dst[:n], src)
        assert torch.all(dst[n:] == 1234)


@pytest.mark.parametrize("as_given", [False, True])
@pytest.mark.parametrize("schedule", ["static", "dynamic", "dynamic_xcd"])
def test_grouped_tile_order_deepest_first(pts, schedule, as_given):
    # problems of different depth: by default the deepest come first in the tile
    # order (so they are dealt / claimed first); on request the descriptor order
    ks = [64, 1000, 8, 520, 1000, 136]
    shapes = [(300, 500, k) for k in ks]
    flags = pts.GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN if as_given else 0
    tensors, refs = [], []
    for g, (m, n, k) in enumerate(shapes):
        a_bits = gen.operand_a(m, k, 7, tensor_id=16 + 2 * g, kind="integer")
        b_bits = gen.operand_b(k, n, 7, tensor_id=17 + 2 * g, kind="integer")
        refs.append(oracle.gemm(a_bits, b_bits, m, n, k))
        tensors.append((U.bits_to_device(a_bits), U.bits_to_device(b_bits),
                        torch.full((m, n), float("nan"), dtype=torch.float32, device=U.DEV)))
    with pts.Plan(shapes, torch.float32, (256, 256), schedule, 0, flags) as p:
        buf = torch.zeros(p.trace_bytes() // 4 + 4, dtype=torch.int32, device=U.DEV)
        p.set_trace(buf)
        p.run(tensors)
        torch.cuda.synchronize()
        tiles, _ = pts.decode_trace(buf, p.num_tiles, p.num_workers)
        U.check_counters(schedule, p.counters(), p.num_tiles, p.num_workers)
    for g, ((_, _, d), ref) in enumerate(zip(tensors, refs)):
        U.check_exact(d, ref, f"problem {g} {schedule}")
    # every tile once, reported under its descriptor index
    want = sorted((g, r0, c0) for (g, r0, c0, _, _) in oracle.tile_coords([s[:2] for s in shapes], 256, 256))
    got = sorted(zip(tiles["group"].tolist(), tiles["row0"].tolist(), tiles["col0"].tolist()))
    assert got == want
    # problem of each position, in position order
    by_pos = [int(g) for _, g in sorted(zip(tiles["tile"].tolist(), tiles["group"].tolist()))]
    per_problem = 2 * 2   # 300 x 500 in 256 x 256 tiles
    order = list(range(len(ks))) if as_given else sorted(range(len(ks)), key=lambda g: -((ks[g] + 63) // 64))
    assert by_pos == [g for g in order for _ in range(per_problem)]


def _preset_run(pts, schedule, preset, m=1000, n=1000, k=64):
    """One traced run of an integer-valued problem with the claim counters
    preset, D filled with NaN beforehand."""
    a_bits = gen.operand_a(m, k, 17, kind="integer")
    b_bits = gen.operand_b(k, n, 17, kind="integer")
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    d = torch.full((m, n), float("nan"), dtype=torch.float32, device=U.DEV)
    with pts.Plan([(m, n, k)], torch.float32, (256, 256), schedule) as p:
        buf = torch.zeros(p.trace_bytes() // 4 + 4, dtype=torch.int32, device=U.DEV)
        p.set_trace(buf)
        p.preset_claims(preset)
        p.run([(a, b, d)])
        torch.cuda.synchronize()
        tiles, workers = pts.decode_trace(buf, p.num_tiles, p.num_workers)
        counters = p.counters()
        nt, nw = p.num_tiles, p.num_workers
    return d.cpu().double().numpy(), ref, tiles.copy(), workers.copy(), counters, nt, nw


def test_claim_counter_preset_to_tile_count_writes_nothing(pts):
    """The counter starts at T: every worker's first claim is the failed request
    ("Advanced scheduling: Cluster Launch Control", section "One CLC request"),
    so every worker leaves at once and D is untouched."""
    d, _, _, workers, counters, nt, nw = _preset_run(pts, "dynamic", 16)
    assert nt == 16
    assert np.all(np.isnan(d)), "a tile was written although no claim succeeded"
    assert workers["tiles"].tolist() == [0] * nw
    # the preset T plus exactly one failed claim per worker; the counters reset
    assert counters[:2] == [0, 0] and counters[2] == nt + nw


def test_claim_counter_preset_to_k_writes_tiles_k_to_t(pts):
    """The counter starts at k = 5: the run processes exactly the tile
    positions 5 .. T-1, each once, and leaves the first five tiles unwritten."""
    k0 = 5
    d, ref, tiles, workers, counters, nt, nw = _preset_run(pts, "dynamic", k0)
    ran = sorted(int(t) for t, w in zip(tiles["tile"], tiles["t_end"]) if w != 0)
    assert ran == list(range(k0, nt))
    assert int(workers["tiles"].sum()) == nt - k0
    assert counters[2] == nt + nw          # k0 preset + (T - k0) tiles + one failed claim per worker
    tiles_m = tiles_n = 4
    for pos in range(nt):
        tm, tn = pos % tiles_m, pos // tiles_m     # the plan's raster: 4 tile rows, walked by column
        blk = d[tm * 256:(tm + 1) * 256, tn * 256:(tn + 1) * 256]
        want = ref[tm * 256:(tm + 1) * 256, tn * 256:(tn + 1) * 256]
        if pos < k0:
            assert np.all(np.isnan(blk)), f"tile at position {pos} was written"
        else:
            assert np.array_equal(blk, want), f"tile at position {pos} is wrong"


def test_xcd_claim_counters_preset_past_their_sequences_write_nothing(pts):
    """Per-XCD counters preset beyond every XCD's sequence: each worker finds
    its own sequence and every other one drained, and leaves at once."""
    d, _, _, workers, counters, nt, nw = _preset_run(pts, "dynamic_xcd", 3)   # 16 tiles: 2 per XCD
    assert np.all(np.isnan(d))
    assert workers["tiles"].tolist() == [0] * nw
    assert counters[:2] == [0, 0]


def test_preset_claims_rejects_static_plans(pts):
    with pts.Plan([(64, 64, 64)], torch.float32, (64, 64), "static") as p:
        with pytest.raises(pts.GemmError):
            p.preset_claims(1)


def test_plans_created_and_destroyed_do_not_leak(pts):
    """500 plans created and destroyed: the device's free memory comes back."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0, _ = torch.cuda.mem_get_info()
    for i in range(500):
        desc = pts.make_desc([(256 + i, 512, 64)] * (1 + i % 8), pts.GEMM_DTYPE_BF16,
                             schedule=i % 3)
        pts.gemm_plan_destroy(pts.gemm_plan_create(desc))
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 >= free0 - (2 << 20), f"free memory fell by {free0 - free1} bytes over 500 plans"


@pytest.mark.parametrize("kernel", [(0, 0), (256, 256, 64, 2, 1, 4, 16)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("schedule", ["dynamic", "dynamic_xcd"])
def test_claim_after_tile_same_d_and_valid_claims(pts, schedule, out_dtype, kernel):
    # Request-ahead off ("Advanced scheduling: Cluster Launch Control", section
    # on overlapping the request with the current computation, as a baseline):
    # the next tile is requested only after the epilogue. D must be bit-identical
    # to the default (the summation order does not depend on who computes a
    # tile), every tile computed once, the claims valid and the counters reset.
    # bf16 output runs the tile loop that loads the next tile during the
    # epilogue (both 256x256 kernels), fp32 output the staged one; the trace is
    # on in every run.
    shapes = [(1000, 1500, 296), (600, 700, 1000), (257, 129, 64)]
    ops = []
    for g, (m, n, k) in enumerate(shapes):
        a = gen.uniform_bf16_torch(m * k, 10 + g, 1, U.DEV).view(m, k)
        b = gen.uniform_bf16_torch(n * k, 10 + g, 2, U.DEV).view(n, k)
        ops.append((a, b))
    outs = {}
    for flags in (0, pts.GEMM_FLAG_CLAIM_AFTER_TILE):
        U.log(f"claim after tile: {schedule} {out_dtype} kernel {kernel} flags {flags}")
        ds = [torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV) for (m, n, _) in shapes]
        with pts.Plan(shapes, out_dtype, kernel, schedule, 0, flags) as p:
            buf = torch.zeros(p.trace_bytes() // 4 + 4, dtype=torch.int32, device=U.DEV)
            p.set_trace(buf)
            for _ in range(2):
                p.run([(a, b, d) for (a, b), d in zip(ops, ds)])
            torch.cuda.synchronize()
            tiles, workers = pts.decode_trace(buf, p.num_tiles, p.num_workers)
            nt, nw, counters = p.num_tiles, p.num_workers, p.counters()
        assert sorted(tiles["tile"].tolist()) == list(range(nt))
        order = np.lexsort((tiles["seq"], tiles["worker"]))
        per_worker = [[] for _ in range(nw)]
        for i in order:
            per_worker[tiles["worker"][i]].append(int(tiles["claim"][i]))
        if schedule == "dynamic":
            oracle.check_dynamic_claims(per_worker, nt)
        else:
            check_xcd_claims(per_worker, (workers["xcc_id"] % 8).tolist(), nt, nw)
        U.check_counters(schedule, counters, nt, nw)
        outs[flags] = [d.cpu() for d in ds]
    for d0, d1 in zip(outs[0], outs[pts.GEMM_FLAG_CLAIM_AFTER_TILE]):
        assert not torch.isnan(d1).any()
        bits = torch.int32 if out_dtype == torch.float32 else torch.int16
        assert torch.equal(d0.view(bits), d1.view(bits))
