"""GPU tests of GEMM_TILE_AUTO: the plan picks the first of 256x256, 256x128
and 128x128 whose tile count reaches 55% of the compute units, else 64x64, and
the result is the oracle's on sampled entries (every tile's corners plus
random ones)."""
from __future__ import annotations

import pytest
import torch

from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _tiles(shapes, tm, tn):
    return sum(-(-m // tm) * -(-n // tn) for (m, n, _k) in shapes if m > 0 and n > 0)


def _expected_tile(shapes, cus):
    for tm, tn in ((256, 256), (256, 128), (128, 128)):
        if 20 * _tiles(shapes, tm, tn) >= 11 * cus:
            return tm, tn
    return 64, 64


@pytest.mark.parametrize("shapes", [
    [(1000, 1000, 264)],                  # 16 tiles of 256, 32 of 256x128, 64 of 128: 64x64
    [(2048, 2048, 520)],                  # 64 of 256, 128 of 256x128, 256 of 128: 128x128
    [(2560, 2500, 264)],                  # 100 of 256, 200 of 256x128: 256x128
    [(3000, 3100, 136)],                  # 156 of 256: 256x256
    [(700, 1500, 200), (900, 300, 72)],   # grouped: the count is over all problems
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_auto_tile_choice_and_parity(pts, shapes, out_dtype):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm, tn = _expected_tile(shapes, cus)
    U.log(f"auto tile {shapes} {out_dtype}: expect {tm}x{tn} on {cus} CUs")
    ops, samples = [], []
    for i, (m, n, k) in enumerate(shapes):
        a = U.device_uniform(m, k, 40 + i, 1)
        b = U.device_uniform(n, k, 40 + i, 2)
        d = torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV)
        ops.append((a, b, d))
        (rows, cols), = U.sample_entries([(m, n)], tm, tn, 100, seed=i)
        samples.append((rows, cols, U.oracle_sampled(40 + i, 1, 2, k, rows, cols)))
    with pts.Plan(shapes, out_dtype, "auto", "dynamic_xcd") as p:
        assert p.num_tiles == _tiles(shapes, tm, tn)
        assert (p.kernel["tile_m"], p.kernel["tile_n"]) == (tm, tn)
        p.run(ops)
        torch.cuda.synchronize()
        U.check_counters("dynamic_xcd", p.counters(), p.num_tiles, p.num_workers)
    for i, ((m, n, k), (_, _, d), (rows, cols, ref)) in enumerate(zip(shapes, ops, samples)):
        U.check_sampled(d, rows, cols, ref, k, f"auto tile problem {i} {(m, n, k)}")
