"""The stage hand-off through LDS arrive counters (the pages' FusedMerge and
Merge barrier layouts) against the oracle and against the workgroup-barrier
form, which must give the same bits.

Cases stress what the counters track: many tiles per worker (the counts run on
across tiles, with odd and even k-tile counts), edge tiles (every wave loads)
mixed with full tiles (half the waves load for two), K tails, the rotated k
order, grouped problems of unequal K, and every schedule.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import pts_inputs as gen
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DEFAULT = (256, 256, 64, 2, 1, 8, 16)
SCHEDULES = ["static", "dynamic", "dynamic_xcd", "nonpersistent"]
MODES = {"fused": 1, "merged": 2}


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _padded_ld(k):
    return max(8, (k + 7) // 8 * 8)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("shape,workers", [
    ((2048, 2048, 200), 7),      # 64 full tiles, 4 k-tiles with a tail, ~9 tiles per worker
    ((2000, 1900, 136), 5),      # edge tiles in both directions, 3 k-tiles (odd), 13 tiles per worker
    ((1000, 1000, 1000), 0),     # 16 tiles, one per worker
    ((300, 200, 8), 0),          # one k-tile, one partial tile
    ((513, 257, 2000), 3),       # edge tiles, 32 k-tiles
    ((2304, 2304, 1000), 0),     # 81 tiles: rotated k order, the partial k-tile mid-loop
])
def test_integer_exact_and_equal_to_barrier(pts, mode, shape, workers):
    m, n, k = shape
    lda = ldb = _padded_ld(k)
    a_bits = gen.operand_a(m, k, 21, lda=lda, kind="integer")
    b_bits = gen.operand_b(k, n, 21, ldb=ldb, kind="integer")
    ref = oracle.gemm(a_bits, b_bits, m, n, k, lda=lda, ldb=ldb)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    for out_dtype in (torch.float32, torch.bfloat16):
        for sched in SCHEDULES:
            nw = workers if sched != "nonpersistent" else 0
            U.log(f"stage flags {mode} {shape} workers {nw} {out_dtype} {sched}")
            d, counters, info = U.run_single(m, n, k, a, b, out_dtype, sched, tile=DEFAULT, lda=lda, ldb=ldb,
                                             num_workers=nw, flags=MODES[mode])
            U.check_counters(sched, counters, *info)
            U.check_exact(d[:m, :n], ref, f"{mode} {shape} {sched}")


@pytest.mark.parametrize("mode", list(MODES))
def test_random_inputs_bitwise_equal_to_barrier(pts, mode):
    m, n, k = 1500, 1300, 1000
    a_bits = gen.operand_a(m, k, 31)
    b_bits = gen.operand_b(k, n, 31)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    for out_dtype in (torch.float32, torch.bfloat16):
        for sched in SCHEDULES:
            U.log(f"stage flags random {mode} {out_dtype} {sched}")
            base, _, _ = U.run_single(m, n, k, a, b, out_dtype, sched, tile=DEFAULT)
            d, counters, info = U.run_single(m, n, k, a, b, out_dtype, sched, tile=DEFAULT, flags=MODES[mode])
            U.check_counters(sched, counters, *info)
            assert torch.equal(base, d), f"{mode} {sched} differs from the barrier form"
            tol = (2e-3 if out_dtype == torch.float32 else 1e-2) * np.sqrt(k)
            err = np.abs(d.double().cpu().numpy() - ref).max()
            assert err <= tol, (err, tol)


@pytest.mark.parametrize("mode", list(MODES))
def test_grouped_variable_k(pts, mode):
    rng = np.random.default_rng(41)
    problems = [(int(rng.integers(1, 700)), int(rng.integers(1, 700)), int(rng.choice([8, 64, 136, 520, 1000])))
                for _ in range(12)]
    shapes, tensors, refs = [], [], []
    for g, (m, n, k) in enumerate(problems):
        a_bits = gen.operand_a(m, k, 41, lda=_padded_ld(k), tensor_id=16 + 2 * g, kind="integer")
        b_bits = gen.operand_b(k, n, 41, ldb=_padded_ld(k), tensor_id=17 + 2 * g, kind="integer")
        refs.append(oracle.gemm(a_bits, b_bits, m, n, k, lda=_padded_ld(k), ldb=_padded_ld(k)))
        shapes.append((m, n, k, _padded_ld(k), _padded_ld(k), 0))
        tensors.append((U.bits_to_device(a_bits), U.bits_to_device(b_bits),
                        torch.full((m, n), float("nan"), dtype=torch.float32, device=U.DEV)))
    for sched in SCHEDULES:
        U.log(f"stage flags grouped {mode} {sched}")
        with pts.Plan(shapes, torch.float32, DEFAULT, sched, 0, MODES[mode]) as p:
            p.run(tensors)
            torch.cuda.synchronize()
            counters = p.counters()
            U.check_counters(sched, counters, p.num_tiles, p.num_workers)
        for (m, n, k), (_, _, d), ref in zip(problems, tensors, refs):
            U.check_exact(d, ref, f"grouped {mode} {(m, n, k)} {sched}")


@pytest.mark.parametrize("mode", list(MODES))
def test_waits_are_bounded(pts, mode):
    # Forced from the host: every full target asks for one arrival too many, so
    # every wave's first wait runs out. The kernel must still end, promptly, with
    # one expired wait counted per wave; a normal plan afterwards runs clean.
    import time
    m = n = k = 512
    a = torch.zeros((m, k), dtype=torch.bfloat16, device=U.DEV)
    b = torch.zeros((n, k), dtype=torch.bfloat16, device=U.DEV)
    d = torch.empty((m, n), dtype=torch.float32, device=U.DEV)
    U.log(f"bounded stage-flag waits {mode}")
    flags = MODES[mode] | pts.GEMM_FLAG_DEBUG_STAGE_FLAG_STALL
    with pts.Plan([(m, n, k)], torch.float32, DEFAULT, "static", 0, flags) as p:
        t0 = time.perf_counter()
        p.run([(a, b, d)])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        counters = p.counters()
        waves = p.num_workers * 8
    assert counters[4] == waves, counters
    assert elapsed < 5.0, elapsed
    d.fill_(float("nan"))
    with pts.Plan([(m, n, k)], torch.float32, DEFAULT, "static", 0, MODES[mode]) as p:
        p.run([(a, b, d)])
        torch.cuda.synchronize()
        assert p.counters()[4] == 0
    assert torch.count_nonzero(d).item() == 0
