"""GPU tests: plans running at the same time on separate streams.

A dynamic plan's claim counters are device memory the plan owns, and the
kernel puts them back to zero at the end of every run, so plans launched on
separate streams run side by side without seeing each other's claims. A
persistent launch holds every compute unit it can, so the workers of a launch
queued behind another typically start only as the first one's workers leave:
the late-start case that claiming from a shared pool absorbs ("Advanced
scheduling: Cluster Launch Control", section on the limits of the static
persistent scheduler). Each plan first runs alone, checked against the oracle
on sampled entries; then all plans run several times concurrently, every
output is compared bit for bit with the run alone (a tile's summation order
depends on its position only), and each plan's counters must show complete,
reset runs.
"""
from __future__ import annotations

import pytest
import torch

import pts_inputs as gen
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

# (problems, output dtype, schedule): both dynamic forms beside a static plan,
# a grouped plan among them, bf16 and fp32 outputs, ragged edges and a k tail
CASES = [
    ([(2048, 2048, 1024)], torch.bfloat16, "dynamic_xcd"),
    ([(1536, 2560, 776)], torch.float32, "dynamic"),
    ([(1000, 1500, 296), (600, 700, 1000), (257, 129, 64)], torch.bfloat16, "static"),
    ([(3000, 1100, 520)], torch.bfloat16, "dynamic_xcd"),
]
RUNS = 4


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _tensor_ids(shapes, g):
    return gen.group_tensor_ids(g) if len(shapes) > 1 else (gen.TENSOR_A, gen.TENSOR_B)


def _operands(shapes, seed):
    ops = []
    for g, (m, n, k) in enumerate(shapes):
        ta, tb = _tensor_ids(shapes, g)
        ops.append((gen.uniform_bf16_torch(m * k, seed, ta, U.DEV).view(m, k),
                    gen.uniform_bf16_torch(n * k, seed, tb, U.DEV).view(n, k)))
    return ops


def _blank(shapes, out_dtype):
    return [torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV) for (m, n, _) in shapes]


def _bits(d):
    return d.view(torch.int16 if d.dtype == torch.bfloat16 else torch.int32)


def test_plans_on_separate_streams_run_concurrently(pts):
    plans, ops, refs = [], [], []
    try:
        for i, (shapes, out_dtype, schedule) in enumerate(CASES):
            seed = 40 + i
            U.log(f"concurrent plans: case {i} alone ({schedule}, {out_dtype}, {len(shapes)} problems)")
            o = _operands(shapes, seed)
            p = pts.Plan(shapes, out_dtype, (0, 0), schedule)
            plans.append(p)
            ds = _blank(shapes, out_dtype)
            p.run([(a, b, d) for (a, b), d in zip(o, ds)])
            torch.cuda.synchronize()
            samples = U.sample_entries([(m, n) for (m, n, _) in shapes], 256, 256, 128, seed=i)
            for g, ((m, n, k), d, (rows, cols)) in enumerate(zip(shapes, ds, samples)):
                ta, tb = _tensor_ids(shapes, g)
                ref = U.oracle_sampled(seed, ta, tb, k, rows, cols)
                U.check_sampled(d, rows, cols, ref, k, f"case {i} problem {g} alone")
            ops.append(o)
            refs.append(ds)

        streams = [torch.cuda.Stream() for _ in CASES]
        outs = [[_blank(shapes, out_dtype) for _ in range(RUNS)] for (shapes, out_dtype, _) in CASES]
        torch.cuda.synchronize()
        U.log(f"concurrent plans: {len(CASES)} plans x {RUNS} runs on {len(CASES)} streams")
        for r in range(RUNS):
            for i, p in enumerate(plans):
                p.run([(a, b, d) for (a, b), d in zip(ops[i], outs[i][r])], streams[i])
        torch.cuda.synchronize()

        for i, p in enumerate(plans):
            for r in range(RUNS):
                for g, (d, ref) in enumerate(zip(outs[i][r], refs[i])):
                    assert torch.equal(_bits(d), _bits(ref)), f"case {i} run {r} problem {g} differs from its run alone"
            U.check_counters(CASES[i][2], p.counters(), p.num_tiles, p.num_workers)
    finally:
        for p in plans:
            p.close()
