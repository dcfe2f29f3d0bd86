"""GPU parity: the HIP GEMM against the oracle on the same seeded inputs.

Bars (the tolerance is written here, per case):
* integer-valued inputs -- bit-exact: fp32 output equals the oracle's exact
  sum, bf16 output equals the oracle's round-to-nearest-even of it;
* uniform[-1, 1] inputs -- max |D - ref| <= 2e-3 sqrt(K) (fp32 output) or
  1e-2 sqrt(K) (bf16 output): over every element at oracle-sized shapes, over
  every element of D for the 8192^3 and 5000x7000x3000 configurations, over
  every element of every edge tile plus one full tile per problem for the
  grouped configuration, and over 64 whole tiles of the 16384^2 x 8192 one;
* static, dynamic, per-XCD dynamic and non-persistent schedules -- bitwise
  identical D (same tile body).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import pts_inputs as gen
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCHEDULES = ("static", "dynamic", "dynamic_xcd", "nonpersistent")
PERSISTENT = SCHEDULES[:3]   # the schedules that take a worker count


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _operands(m, n, k, seed, kind="uniform", lda=0, ldb=0):
    a_bits = gen.operand_a(m, k, seed, lda=lda or None, kind=kind) if m else np.zeros((0, max(lda, k, 8)), np.uint16)
    b_bits = gen.operand_b(k, n, seed, ldb=ldb or None, kind=kind) if n else np.zeros((0, max(ldb, k, 8)), np.uint16)
    return a_bits, b_bits


def _padded_ld(k):
    return max(8, (k + 7) // 8 * 8)


# ---------------------------------------------------------------------------
# Config 1: 256^3, fp32 output, 64x64 tiles (16 tiles) -- full oracle
# ---------------------------------------------------------------------------

def test_config1_256_cube_fp32_64x64(pts):
    m = n = k = 256
    a_bits, b_bits = _operands(m, n, k, 0)
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    outs = {}
    for sched in SCHEDULES:
        U.log(f"config1 256^3 fp32 tile 64x64 schedule={sched}")
        d, counters, (tiles, workers) = U.run_single(m, n, k, a, b, torch.float32, sched, tile=(64, 64))
        assert (tiles, workers) == (16, 16)
        err = U.check_close(d, ref, k, f"config1 {sched}")
        U.log(f"  max err {err:.3g} (tol {U.tol_for(torch.float32, k):.3g})")
        outs[sched] = d
    for sched in SCHEDULES[1:]:
        assert torch.equal(outs["static"], outs[sched])


# ---------------------------------------------------------------------------
# Integer-exact sweep over edge sizes, every tile size, both output types
# ---------------------------------------------------------------------------

SWEEP = [(1, 1, 1), (7, 7, 7), (63, 65, 64), (64, 64, 64), (65, 63, 65), (127, 129, 128), (128, 128, 127),
         (129, 127, 129), (255, 257, 256), (256, 256, 255), (257, 255, 257), (1000, 1000, 1000),
         (1, 1000, 63), (1000, 1, 129), (257, 1, 1), (1, 257, 257), (300, 200, 8), (33, 520, 1000)]


# every built kernel: (tile_m, tile_n, tile_k, stages, load path, waves[, mfma])
KERNELS = [(64, 64, 64, 2, 1, 4), (128, 128, 64, 2, 1, 4), (256, 256, 64, 2, 1, 8, 16), (256, 256, 64, 2, 1, 4, 16),
           (256, 128, 64, 2, 1, 8, 16)]


@pytest.mark.parametrize("tile", KERNELS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_integer_exact_sweep(pts, tile, out_dtype):
    for (m, n, k) in SWEEP:
        lda = ldb = _padded_ld(k)
        a_bits, b_bits = _operands(m, n, k, 3, kind="integer", lda=lda, ldb=ldb)
        ref = oracle.gemm(a_bits, b_bits, m, n, k, lda=lda, ldb=ldb)
        a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
        for sched in SCHEDULES:
            U.log(f"integer sweep {(m, n, k)} tile {tile} {out_dtype} {sched}")
            d, _, _ = U.run_single(m, n, k, a, b, out_dtype, sched, tile=tile, lda=lda, ldb=ldb)
            U.check_exact(d[:m, :n], ref, f"{(m, n, k)} tile {tile} {sched}")


_ROTATED_CASE = {}


def _rotated_case():
    # 2304 x 2304 x 1000: 81 tiles of 256 (1296 of 64), so tiles past the first
    # 32 positions start their k loop part-way through K, and the partial last
    # k-tile (K = 15 * 64 + 40) is visited in the middle of the loop
    if not _ROTATED_CASE:
        m = n = 2304
        k = 1000
        lda = ldb = _padded_ld(k)
        a_bits, b_bits = _operands(m, n, k, 11, kind="integer", lda=lda, ldb=ldb)
        _ROTATED_CASE.update(m=m, n=n, k=k, lda=lda, ldb=ldb, a_bits=a_bits, b_bits=b_bits,
                             ref=oracle.gemm(a_bits, b_bits, m, n, k, lda=lda, ldb=ldb))
    return _ROTATED_CASE


@pytest.mark.parametrize("tile", KERNELS)
def test_k_tail_first_in_rotated_order(pts, tile):
    """256 tile positions and an odd number of k-tiles: the tiles' rotated k
    orders then start at every k-tile, the partial last one included, which is
    then the first k-tile the loop loads (its k >= K part must be zeroed before
    the first fragment reads). For 256x256 tiles also 1156 positions (more than
    four rounds of the chip, where tile rows share their k start): some k
    orders start at the partial k-tile there too. Every tile is checked at its
    four corners."""
    bm = tile[0]
    k = 520  # 9 k-tiles of 64 or 17 of 32; the last holds 8 values of k
    seed = 23
    for edge_tiles in ((16, 34) if bm == 256 else (16,)):
        m = n = edge_tiles * bm
        a = U.device_uniform(m, k, seed, 1)
        b = U.device_uniform(n, k, seed, 2)
        (rows, cols), = U.sample_entries([(m, n)], bm, bm, 300, seed=3)
        ref = U.oracle_sampled(seed, 1, 2, k, rows, cols)
        for sched in ("static", "dynamic_xcd"):
            U.log(f"k tail first tile {tile} {sched} {m}x{n}x{k}")
            d, _, _ = U.run_single(m, n, k, a, b, torch.float32, sched, tile=tile)
            U.check_sampled(d, rows, cols, ref, k, f"k tail first tile {tile} {sched} {m}x{n}")
        del a, b, d


@pytest.mark.parametrize("tile", KERNELS)
def test_rotated_k_order_with_k_tail(pts, tile):
    c = _rotated_case()
    a, b = U.bits_to_device(c["a_bits"]), U.bits_to_device(c["b_bits"])
    for out_dtype in (torch.float32, torch.bfloat16):
        for sched in SCHEDULES:
            U.log(f"rotated k order tile {tile} {out_dtype} {sched}")
            d, _, _ = U.run_single(c["m"], c["n"], c["k"], a, b, out_dtype, sched, tile=tile, lda=c["lda"],
                                   ldb=c["ldb"])
            U.check_exact(d[:c["m"], :c["n"]], c["ref"], f"rotated tile {tile} {out_dtype} {sched}")


# ---------------------------------------------------------------------------
# Random inputs, ragged medium shapes, full oracle; D padding untouched
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(600, 700, 300), (257, 129, 1000), (1000, 1000, 64), (513, 257, 2000),
                                   (40, 3000, 100)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("tile", KERNELS)
def test_random_ragged_full_oracle(pts, shape, out_dtype, tile):
    m, n, k = shape
    lda, ldb, ldd = _padded_ld(k) + 16, _padded_ld(k) + 8, n + 5
    a_bits, b_bits = _operands(m, n, k, 5, lda=lda, ldb=ldb)
    ref = oracle.gemm(a_bits, b_bits, m, n, k, lda=lda, ldb=ldb)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    outs = {}
    for sched in SCHEDULES:
        U.log(f"ragged {shape} {out_dtype} {sched}")
        d = torch.full((m + 3, ldd), 7.0, dtype=out_dtype, device=U.DEV)
        U.run_single(m, n, k, a, b, out_dtype, sched, tile=tile, lda=lda, ldb=ldb, ldd=ldd, d=d)
        U.check_close(d[:m, :n], ref, k, f"{shape} {sched}")
        assert torch.all(d[:m, n:] == 7.0), "row padding of D was written"
        assert torch.all(d[m:] == 7.0), "rows past M were written"
        outs[sched] = d
    for sched in SCHEDULES[1:]:
        assert torch.equal(outs["static"], outs[sched])


def test_identity_reproduces_a(pts):
    m, k = 300, 256
    a_bits = gen.operand_a(m, k, 8)
    b_bits = np.zeros((k, k), np.uint16)
    np.fill_diagonal(b_bits, 0x3F80)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    for sched in SCHEDULES:
        d, _, _ = U.run_single(m, k, k, a, b, torch.bfloat16, sched)
        assert np.array_equal(U.device_to_bits(d), a_bits), "A . I != A (bf16 output)"


def test_ones_closed_form_rne(pts):
    # K = 3000 and 3016 are ties in bf16; ties-to-even gives 3008 for both.
    for k, want in ((3000, 3008.0), (3016, 3008.0), (3001, 3008.0), (64, 64.0)):
        ld = _padded_ld(k)
        a = torch.zeros((70, ld), dtype=torch.bfloat16, device=U.DEV)
        a[:, :k] = 1
        b = torch.zeros((90, ld), dtype=torch.bfloat16, device=U.DEV)
        b[:, :k] = 1
        d, _, _ = U.run_single(70, 90, k, a, b, torch.bfloat16, "dynamic", lda=ld, ldb=ld)
        assert torch.all(d.float() == want), f"K={k}"
        d32, _, _ = U.run_single(70, 90, k, a, b, torch.float32, "static", lda=ld, ldb=ld)
        assert torch.all(d32 == float(k))


# ---------------------------------------------------------------------------
# Degenerate shapes
# ---------------------------------------------------------------------------

def test_k_zero_writes_zeros(pts):
    for sched in SCHEDULES:
        d, _, (tiles, _) = U.run_single(300, 200, 0, None, None, torch.float32, sched)
        assert tiles == 2
        assert torch.all(d == 0)


def test_m_or_n_zero_is_a_noop(pts):
    for (m, n) in ((0, 100), (100, 0)):
        d = torch.full((max(m, 1), max(n, 1)), 5.0, device=U.DEV)
        a = torch.zeros((max(m, 1), 64), dtype=torch.bfloat16, device=U.DEV)
        b = torch.zeros((max(n, 1), 64), dtype=torch.bfloat16, device=U.DEV)
        _, _, (tiles, workers) = U.run_single(m, n, 64, a, b, torch.float32, "dynamic", d=d)
        assert tiles == 0 and workers == 0
        assert torch.all(d == 5.0)


def test_leading_dimensions_at_the_32_bit_offset_limit(pts):
    # A tile's load offsets are 32-bit byte offsets from its origin; the plan
    # accepts leading dimensions up to 255 * ld * 2 + (k + 8) * 2 < 2^31. Use the
    # largest such ld (about 2.5 GB per operand) with two tile rows / columns,
    # so the second tile's rows sit just under the limit.
    k = 64
    ld = ((2**31 - 1 - (k + 8) * 2) // (255 * 2)) // 8 * 8
    m = n = 300
    a_bits, b_bits = _operands(m, n, k, 9, kind="integer")
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    for which in ("a", "b"):
        U.log(f"leading dimension {ld} on {which}")
        big = torch.zeros((m, ld), dtype=torch.bfloat16, device=U.DEV)
        if which == "a":
            big[:, :k] = U.bits_to_device(a_bits)
            a, b, lda, ldb = big, U.bits_to_device(b_bits), ld, 0
        else:
            big[:, :k] = U.bits_to_device(b_bits)
            a, b, lda, ldb = U.bits_to_device(a_bits), big, 0, ld
        for sched in ("static", "dynamic_xcd"):
            d, _, (tiles, _) = U.run_single(m, n, k, a, b, torch.float32, sched, lda=lda, ldb=ldb)
            assert tiles == 4
            U.check_exact(d, ref, f"ld {ld} on {which} {sched}")
        del big
        torch.cuda.empty_cache()
    with pytest.raises(pts.GemmError):
        pts.gemm_plan_create(pts.make_desc([(m, n, k, ld + 8, 0, 0)]))


def test_tile_reuse_does_not_accumulate_across_tiles(pts):
    # one worker runs every tile: each tile's accumulators must restart at zero
    m, n, k = 512, 512, 128
    a_bits, b_bits = _operands(m, n, k, 13, kind="integer")
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    for sched in PERSISTENT:
        d, _, (tiles, workers) = U.run_single(m, n, k, a, b, torch.float32, sched, tile=(128, 128), num_workers=1)
        assert (tiles, workers) == (16, 1)
        U.check_exact(d, ref, f"single worker {sched}")


@pytest.mark.parametrize("tile,out_dtype", [((256, 256, 64, 2, 1, 8, 16), torch.bfloat16),
                                            ((256, 256, 64, 2, 1, 4, 16), torch.bfloat16),
                                            ((256, 256, 64, 2, 1, 8, 16), torch.float32),
                                            ((256, 128, 64, 2, 1, 8, 16), torch.float32)])
def test_few_workers_many_tiles(pts, tile, out_dtype):
    # Five workers take many tiles (full and edge ones in turn, a partial last
    # k-tile, k order rotated past the first 32 positions): the tile loop that
    # issues each next tile's first two stages before this tile's stores and
    # then waits for the first stage only, on the 16x16 kernels that run it
    # (bf16 output on both 256x256 kernels, fp32 output on the two-wave ones),
    # every schedule that takes a worker count.
    m, n, k = 1800, 2100, 1000
    lda = ldb = _padded_ld(k)
    a_bits, b_bits = _operands(m, n, k, 17, kind="integer", lda=lda, ldb=ldb)
    ref = oracle.gemm(a_bits, b_bits, m, n, k, lda=lda, ldb=ldb)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    for sched in PERSISTENT:
        U.log(f"few workers, many tiles: tile {tile} {out_dtype} {sched}")
        d, counters, (tiles, workers) = U.run_single(m, n, k, a, b, out_dtype, sched, tile=tile, lda=lda,
                                                     ldb=ldb, num_workers=5)
        assert (tiles, workers) == ((72 if tile[1] == 256 else 136), 5)
        U.check_exact(d[:m, :n], ref, f"5 workers tile {tile} {sched}")
        U.check_counters(sched, counters, tiles, workers)


def test_more_workers_than_tiles(pts):
    m, n, k = 100, 100, 64
    a_bits, b_bits = _operands(m, n, k, 2, kind="integer")
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    for sched in PERSISTENT:
        d, counters, (tiles, workers) = U.run_single(m, n, k, a, b, torch.float32, sched, tile=(64, 64),
                                                     num_workers=9)
        assert (tiles, workers) == (4, 9)
        U.check_exact(d, ref, f"9 workers {sched}")


# ---------------------------------------------------------------------------
# Grouped problems, oracle-sized, full oracle
# ---------------------------------------------------------------------------

def test_grouped_small_full_oracle(pts):
    rng = np.random.default_rng(4)
    shapes = [(int(rng.integers(1, 700)), 300, 200) for _ in range(7)] + [(0, 300, 200), (256, 300, 200)]
    tensors, refs = [], []
    for g, (m, n, k) in enumerate(shapes):
        ta, tb = gen.group_tensor_ids(g)
        a_bits = gen.operand_a(m, k, 1, tensor_id=ta) if m else np.zeros((1, k), np.uint16)
        b_bits = gen.operand_b(k, n, 1, tensor_id=tb)
        refs.append(oracle.gemm(a_bits, b_bits, m, n, k))
        tensors.append((U.bits_to_device(a_bits), U.bits_to_device(b_bits),
                        torch.full((max(m, 1), n), float("nan"), dtype=torch.bfloat16, device=U.DEV)))
    outs = {}
    for sched in SCHEDULES:
        U.log(f"grouped small {sched}")
        for (_, _, d) in tensors:
            d.fill_(float("nan"))
        with pts.Plan(shapes, torch.bfloat16, schedule=sched) as p:
            assert p.num_tiles == sum(-(-m // 256) * 2 for (m, _, _) in shapes)
            p.run(tensors)
            torch.cuda.synchronize()
        for g, ((m, n, k), (_, _, d)) in enumerate(zip(shapes, tensors)):
            if m:
                U.check_close(d[:m], refs[g], k, f"group {g} {sched}")
        outs[sched] = [d.clone() for (_, _, d) in tensors]
    for sched in SCHEDULES[1:]:
        for x, y in zip(outs["static"], outs[sched]):
            assert torch.equal(x.nan_to_num(0.0), y.nan_to_num(0.0))


@pytest.mark.parametrize("out_dtype,num_workers", [(torch.float32, 0), (torch.float32, 3), (torch.bfloat16, 3)])
def test_grouped_variable_k_full_oracle(pts, out_dtype, num_workers):
    # per-problem K (tiles of unequal cost), ragged M, N and K, a K = 0 and a
    # K = 1 problem; with 3 workers the tiles of every K follow each other on a
    # worker, so a tile with no k-tile (nothing loaded, only stores) sits
    # between tiles whose first stages load during the previous epilogue
    rng = np.random.default_rng(6)
    shapes = [(int(rng.integers(1, 400)), int(rng.integers(1, 400)), int(rng.integers(1, 40)) * 8 + int(rng.integers(0, 8)))
              for _ in range(9)] + [(300, 200, 0), (257, 129, 1)]
    tensors, refs = [], []
    for g, (m, n, k) in enumerate(shapes):
        ta, tb = gen.group_tensor_ids(g)
        ld = _padded_ld(k)
        a_bits = gen.operand_a(m, k, 2, tensor_id=ta, lda=ld)
        b_bits = gen.operand_b(k, n, 2, tensor_id=tb, ldb=ld)
        refs.append(oracle.gemm(a_bits, b_bits, m, n, k, lda=ld, ldb=ld))
        tensors.append((U.bits_to_device(a_bits), U.bits_to_device(b_bits),
                        torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV)))
    plan_shapes = [(m, n, k, _padded_ld(k), _padded_ld(k), 0) for (m, n, k) in shapes]
    outs = {}
    for sched in (SCHEDULES if num_workers == 0 else PERSISTENT):
        U.log(f"grouped variable K {sched} {out_dtype} workers {num_workers}")
        for (_, _, d) in tensors:
            d.fill_(float("nan"))
        with pts.Plan(plan_shapes, out_dtype, schedule=sched, num_workers=num_workers) as p:
            p.run(tensors)
            torch.cuda.synchronize()
            U.check_counters(sched, p.counters(), p.num_tiles, p.num_workers)
        for g, ((m, n, k), (_, _, d)) in enumerate(zip(shapes, tensors)):
            U.check_close(d, refs[g], max(k, 1), f"group {g} {(m, n, k)} {sched}")
        outs[sched] = [d.clone() for (_, _, d) in tensors]
    for sched in list(outs)[1:]:
        for x, y in zip(outs["static"], outs[sched]):
            assert torch.equal(x, y)


# ---------------------------------------------------------------------------
# Full-size configurations: every element of D (8192^3, 5000x7000x3000) or of
# whole tiles (grouped, 16384^2 x 8192) against the oracle
# ---------------------------------------------------------------------------

def _host_uniform(rows, cols, seed, tid, first_row=0):
    """Rows first_row .. first_row+rows-1 of a (.. x cols) uniform operand, as bits."""
    return gen.uniform_bf16_bits(seed, tid, rows * cols, start=first_row * cols).reshape(rows, cols)


def _single_full(pts, m, n, k, out_dtype, seed=0):
    """All four schedules, bitwise equal to each other; then every element of D
    against the oracle's full product on the same seeded operands."""
    a_bits = _host_uniform(m, k, seed, gen.TENSOR_A)
    b_bits = _host_uniform(n, k, seed, gen.TENSOR_B)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    first = None
    for sched in SCHEDULES:
        U.log(f"full {m}x{n}x{k} {out_dtype} {sched}")
        d, counters, (tiles, workers) = U.run_single(m, n, k, a, b, out_dtype, sched)
        U.check_counters(sched, counters, tiles, workers)
        if first is None:
            first = d
        else:
            assert torch.equal(first, d), f"{sched} differs from static"
            del d
    U.check_against_fp32_matmul(first, a, b, k, f"{m}x{n}x{k}")
    del a, b
    U.log(f"  oracle: full {m}x{n}x{k} product on {oracle.max_threads()} host threads")
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    err = U.check_close(first, ref, k, f"{m}x{n}x{k} every element")
    U.log(f"  every element: max |D - oracle| = {err:.3g} (tol {U.tol_for(out_dtype, k):.3g})")


def test_generator_on_device_matches_host(pts):
    t = gen.uniform_bf16_torch(1 << 20, 0, gen.TENSOR_A, U.DEV)
    assert np.array_equal(U.device_to_bits(t), gen.uniform_bf16_bits(0, gen.TENSOR_A, 1 << 20))


@pytest.mark.timeout(900)
def test_config2_8192_cube_bf16_every_element(pts):
    _single_full(pts, 8192, 8192, 8192, torch.bfloat16)


@pytest.mark.timeout(600)
def test_config3_ragged_5000x7000x3000_fp32_every_element(pts):
    _single_full(pts, 5000, 7000, 3000, torch.float32)


def _check_blocks(d, blocks, seed, a_tid, b_tid, k, what):
    """Every element of each listed block (r0, r1, c0, c1) of D against the
    oracle's product of A's rows r0..r1-1 and B's columns c0..c1-1 (regenerated
    on the host from the same streams). Returns the largest error."""
    worst = 0.0
    for (r0, r1, c0, c1) in blocks:
        a_rows = _host_uniform(r1 - r0, k, seed, a_tid, first_row=r0)
        b_cols = _host_uniform(c1 - c0, k, seed, b_tid, first_row=c0)
        ref = oracle.gemm(a_rows, b_cols, r1 - r0, c1 - c0, k)
        worst = max(worst, U.check_close(d[r0:r1, c0:c1], ref, k, f"{what} block {(r0, r1, c0, c1)}"))
    return worst


@pytest.mark.timeout(600)
def test_config4_grouped_64_problems_whole_tiles(pts):
    """Every edge tile (the last tile row of each problem whose M_g is not a
    multiple of 256, all 16 tile columns) and one full tile per problem (tile
    column g mod 16 of the first full tile row), every element, against the
    oracle."""
    seed, n, k, bm, bn = 0, 4096, 4096, 256, 256
    ms = gen.grouped_m_draw(seed)
    shapes = [(m, n, k) for m in ms]
    tensors = []
    for g, m in enumerate(ms):
        ta, tb = gen.group_tensor_ids(g)
        tensors.append((U.device_uniform(m, k, seed, ta), U.device_uniform(n, k, seed, tb),
                        torch.empty((m, n), dtype=torch.bfloat16, device=U.DEV)))
    first = None
    for sched in SCHEDULES:
        U.log(f"config4 grouped {sched} sum(M)={sum(ms)}")
        with pts.Plan(shapes, torch.bfloat16, schedule=sched) as p:
            p.run(tensors)
            torch.cuda.synchronize()
            U.check_counters(sched, p.counters(), p.num_tiles, p.num_workers)
        if first is None:
            first = [t[2].clone() for t in tensors]
        else:
            for g, (x, t) in enumerate(zip(first, tensors)):
                assert torch.equal(x, t[2]), f"{sched} differs from static in problem {g}"
    del tensors
    worst, edge_tiles, full_tiles = 0.0, 0, 0
    for g, m in enumerate(ms):
        ta, tb = gen.group_tensor_ids(g)
        blocks = []
        if m % bm:
            r0 = m - m % bm
            blocks.append((r0, m, 0, n))
            edge_tiles += n // bn
        if m >= bm:
            c0 = (g % (n // bn)) * bn
            blocks.append((0, bm, c0, c0 + bn))
            full_tiles += 1
        U.log(f"  oracle: problem {g} (M={m}) blocks {blocks}")
        worst = max(worst, _check_blocks(first[g], blocks, seed, ta, tb, k, f"config4 problem {g}"))
    U.log(f"  {edge_tiles} edge tiles and {full_tiles} full tiles, every element: max err {worst:.3g}")
    assert full_tiles >= sum(1 for m in ms if m >= bm)


@pytest.mark.timeout(600)
def test_config5_with_concurrent_copy_whole_tiles(pts):
    """16384^2 x 8192 while an int16 copy holds 64 CUs. 64 whole tiles are
    compared with the oracle: 8 from each of the 8 classes of k-loop start
    (position // 32 mod 8, one class per compute die's block of a round),
    spread over the rounds and the tile rows of a raster group."""
    m = n = 16384
    k = 8192
    seed = 0
    bm = bn = 256
    a = U.device_uniform(m, k, seed, gen.TENSOR_A)
    b = U.device_uniform(n, k, seed, gen.TENSOR_B)
    ncopy = 1 << 30
    src = gen.uniform_bf16_torch(ncopy, seed, gen.TENSOR_COPY_SRC, U.DEV).view(torch.int16)
    dst = torch.zeros(ncopy + 64, dtype=torch.int16, device=U.DEV)
    # the copy holds 64 of the compute units while the GEMM runs
    copy_stream = pts.pts_stream_create_cu_masked(64)
    first = None
    try:
        for sched in SCHEDULES:
            U.log(f"config5 {sched} with concurrent copy on 64 CUs")
            dst.zero_()
            d = torch.empty((m, n), dtype=torch.bfloat16, device=U.DEV)
            torch.cuda.synchronize()
            with pts.Plan([(m, n, k)], torch.bfloat16, schedule=sched) as p:
                pts.pts_copy_int16(src, dst, ncopy, 256, copy_stream)
                p.run([(a, b, d)])
                torch.cuda.synchronize()
            assert torch.equal(dst[:ncopy], src), "copy result differs"
            assert torch.all(dst[ncopy:] == 0), "copy wrote past the end"
            if first is None:
                first = d
            else:
                assert torch.equal(first, d), f"{sched} differs from static"
                del d
    finally:
        pts.pts_stream_destroy(copy_stream)
    del a, b, src, dst
    tiles_m, tiles_n = m // bm, n // bn
    blocks, classes = [], set()
    for c in range(8):
        for s in range(8):
            pos = 32 * (8 * ((3 * s + c) % 16) + c) + (5 * s + c) % 32
            classes.add((pos // 32) % 8)
            tm, tn = U.raster_tile(pos, tiles_m, tiles_n, U.band_rows(n, k))
            blocks.append((tm * bm, tm * bm + bm, tn * bn, tn * bn + bn))
    assert classes == set(range(8)) and len(set(blocks)) == 64
    U.log(f"  oracle: 64 whole tiles of 256x256x{k}")
    err = _check_blocks(first, blocks, seed, gen.TENSOR_A, gen.TENSOR_B, k, "config5")
    U.log(f"  64 whole tiles: max err {err:.3g}")


def test_config6_grouped_variable_k_sampled(pts):
    seed, m, n = 0, 1024, 1024
    ks = gen.grouped_k_draw(seed)
    shapes = [(m, n, k) for k in ks]
    tensors = []
    for g, k in enumerate(ks):
        ta, tb = gen.group_tensor_ids(g)
        tensors.append((U.device_uniform(m, k, seed, ta), U.device_uniform(n, k, seed, tb),
                        torch.empty((m, n), dtype=torch.bfloat16, device=U.DEV)))
    samples = U.sample_entries([(m, n)] * len(ks), 256, 256, 32, seed=3)
    refs = []
    for g, ((rows, cols), k) in enumerate(zip(samples, ks)):
        ta, tb = gen.group_tensor_ids(g)
        refs.append(U.oracle_sampled(seed, ta, tb, k, rows, cols))
    outs = {}
    for sched in SCHEDULES:
        U.log(f"config6 grouped variable K {sched} sum(K)={sum(ks)}")
        with pts.Plan(shapes, torch.bfloat16, schedule=sched) as p:
            p.run(tensors)
            torch.cuda.synchronize()
            U.check_counters(sched, p.counters(), p.num_tiles, p.num_workers)
        worst = 0.0
        for g, ((rows, cols), ref, k) in enumerate(zip(samples, refs, ks)):
            worst = max(worst, U.check_sampled(tensors[g][2], rows, cols, ref, k, f"config6 group {g} {sched}"))
        U.log(f"  sampled max err {worst:.3g}")
        outs[sched] = [t[2].clone() for t in tensors]
    for sched in SCHEDULES[1:]:
        for x, y in zip(outs["static"], outs[sched]):
            assert torch.equal(x, y)
