"""GPU tests: a run recorded into a HIP graph (through torch.cuda.CUDAGraph) and
replayed.

gemm_run launches one kernel and nothing else: no memset, no copy, no host
synchronisation; the dynamic schedules' claim counters are put back to zero by
the kernel itself at the end of every run. So a captured run must replay
correctly any number of times. Each test replays the graph several times with
the program's own eager work (a fill of D, an eager run of the same plan into
another buffer) and a synchronisation between the replays, and checks every
replay bit for bit against the eager result, which is itself checked against
the oracle on sampled entries.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from tests import gpu_util as U

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _capture(plan, operands):
    """Record plan.run(operands) into a graph; one eager run on a side stream first."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.run(operands)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(operands)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("schedule", ["static", "dynamic", "dynamic_xcd", "nonpersistent"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_single_problem_replays_match_eager(pts, schedule, out_dtype):
    m, n, k, seed = 1000, 1300, 776, 71
    U.log(f"graph single {schedule} {out_dtype} {m}x{n}x{k}")
    a = U.device_uniform(m, k, seed, 1)
    b = U.device_uniform(n, k, seed, 2)
    eager = torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV)
    replay = torch.full_like(eager, float("nan"))
    with pts.Plan([(m, n, k)], out_dtype, (0, 0), schedule) as p:
        p.run([(a, b, eager)])
        torch.cuda.synchronize()
        (rows, cols), = U.sample_entries([(m, n)], 256, 256, 200, seed=seed)
        ref = U.oracle_sampled(seed, 1, 2, k, rows, cols)
        U.check_sampled(eager, rows, cols, ref, k, f"eager {schedule}")
        g = _capture(p, [(a, b, replay)])
        again = torch.empty_like(eager)
        for i in range(REPLAYS):
            replay.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(replay, eager), f"replay {i}: differs from the eager run"
            again.fill_(float("nan"))
            p.run([(a, b, again)])
            torch.cuda.synchronize()
            assert torch.equal(again, eager), f"eager run after replay {i} differs"
        counters = p.counters()
        U.check_counters(schedule, counters, p.num_tiles, p.num_workers)
        if schedule in ("dynamic", "dynamic_xcd"):
            # eager, the warm-up before capture, then each replay and its eager run
            assert counters[3] == 2 + 2 * REPLAYS, f"{counters[3]} completed dynamic runs"


@pytest.mark.parametrize("schedule", ["static", "dynamic_xcd"])
def test_grouped_replays_match_eager(pts, schedule):
    rng = np.random.default_rng(5)
    shapes = [(int(rng.integers(1, 700)), int(rng.integers(1, 600)), 8 * int(rng.integers(1, 90)))
              for _ in range(12)]
    U.log(f"graph grouped {schedule} {shapes}")
    ops_eager, ops_replay = [], []
    for i, (m, n, k) in enumerate(shapes):
        a = U.device_uniform(m, k, 90 + i, 1)
        b = U.device_uniform(n, k, 90 + i, 2)
        ops_eager.append((a, b, torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=U.DEV)))
        ops_replay.append((a, b, torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=U.DEV)))
    with pts.Plan(shapes, torch.bfloat16, (0, 0), schedule) as p:
        p.run(ops_eager)
        torch.cuda.synchronize()
        for i, ((m, n, k), (_, _, d)) in enumerate(zip(shapes, ops_eager)):
            (rows, cols), = U.sample_entries([(m, n)], 256, 256, 50, seed=i)
            U.check_sampled(d, rows, cols, U.oracle_sampled(90 + i, 1, 2, k, rows, cols), k, f"eager problem {i}")
        g = _capture(p, ops_replay)
        for r in range(REPLAYS):
            for _, _, d in ops_replay:
                d.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for i, ((_, _, de), (_, _, dr)) in enumerate(zip(ops_eager, ops_replay)):
                assert torch.equal(dr, de), f"replay {r}, problem {i}: differs from the eager run"
        counters = p.counters()
        U.check_counters(schedule, counters, p.num_tiles, p.num_workers)
        if schedule == "dynamic_xcd":
            assert counters[3] == 2 + REPLAYS, f"{counters[3]} completed dynamic runs"
