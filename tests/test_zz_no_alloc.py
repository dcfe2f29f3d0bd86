"""GPU test of gemm_run_noalloc, the entry point for callers that cannot
allocate device memory: called through the C ABI, its output must equal
gemm_run's (same descriptor, same operands) bit for bit, on two calls in a
row -- the second with a smaller input -- for every schedule, single and
grouped, and the integer-valued cases must equal the oracle exactly."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import pts_inputs as gen
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCHEDULES = ("static", "dynamic", "dynamic_xcd", "nonpersistent")


@pytest.fixture(scope="module")
def pts():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_tile_scheduling_amd as mod
    return mod


def _sched(pts, name):
    return {"static": pts.GEMM_SCHEDULE_STATIC, "dynamic": pts.GEMM_SCHEDULE_DYNAMIC,
            "dynamic_xcd": pts.GEMM_SCHEDULE_DYNAMIC_XCD, "nonpersistent": pts.GEMM_SCHEDULE_NONPERSISTENT}[name]


def _noalloc_c_abi(pts, desc, operands):
    """gemm_run_noalloc called through ctypes on the library itself."""
    lib = ctypes.CDLL(pts.LIB_PATH)
    fn = lib.gemm_run_noalloc
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.POINTER(pts.GemmDesc), ctypes.POINTER(pts.GemmOperands), ctypes.c_void_p]
    arr = (pts.GemmOperands * len(operands))()
    for i, (a, b, d) in enumerate(operands):
        arr[i] = pts.GemmOperands(a.data_ptr(), b.data_ptr(), d.data_ptr())
    st = fn(ctypes.byref(desc), arr, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == pts.GEMM_OK, pts.gemm_last_error()


def _problems(shapes, seed, kind):
    out = []
    for g, (m, n, k) in enumerate(shapes):
        ta, tb = gen.group_tensor_ids(g) if len(shapes) > 1 else (gen.TENSOR_A, gen.TENSOR_B)
        a_bits = gen.operand_a(m, k, seed, tensor_id=ta, kind=kind)
        b_bits = gen.operand_b(k, n, seed, tensor_id=tb, kind=kind)
        out.append((a_bits, b_bits))
    return out


def _compare(pts, shapes, out_dtype, schedule, seed, kind="integer"):
    bits = _problems(shapes, seed, kind)
    dev = [(U.bits_to_device(a), U.bits_to_device(b)) for (a, b) in bits]
    dtype_d = pts.GEMM_DTYPE_BF16 if out_dtype == torch.bfloat16 else pts.GEMM_DTYPE_F32
    desc = pts.make_desc(shapes, dtype_d, schedule=_sched(pts, schedule))
    d_plan = [torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV) for (m, n, _) in shapes]
    d_free = [torch.full((m, n), float("nan"), dtype=out_dtype, device=U.DEV) for (m, n, _) in shapes]
    plan = pts.gemm_plan_create(desc)
    try:
        pts.gemm_run(plan, [(a, b, d) for (a, b), d in zip(dev, d_plan)])
    finally:
        torch.cuda.synchronize()
        pts.gemm_plan_destroy(plan)
    _noalloc_c_abi(pts, desc, [(a, b, d) for (a, b), d in zip(dev, d_free)])
    torch.cuda.synchronize()
    for g, (x, y) in enumerate(zip(d_plan, d_free)):
        assert torch.equal(x, y), f"problem {g} {schedule}: gemm_run_noalloc differs from gemm_run"
    if kind == "integer":
        for g, ((a, b), d, (m, n, k)) in enumerate(zip(bits, d_free, shapes)):
            U.check_exact(d, oracle.gemm(a, b, m, n, k), f"problem {g} {schedule}")


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_noalloc_matches_gemm_run_twice_second_smaller(pts, schedule):
    U.log(f"no-alloc single {schedule}")
    _compare(pts, [(1000, 900, 520)], torch.float32, schedule, 3)
    _compare(pts, [(300, 200, 136)], torch.float32, schedule, 4)


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_noalloc_grouped_twice_second_smaller(pts, schedule):
    U.log(f"no-alloc grouped {schedule}")
    big = [(700, 600, 200), (256, 512, 64), (0, 100, 64), (1, 1, 8), (900, 300, 1000)] * 4
    _compare(pts, big, torch.bfloat16, schedule, 5)
    _compare(pts, [(130, 70, 72), (64, 64, 64)], torch.bfloat16, schedule, 6)


def test_noalloc_uniform_inputs_full_oracle(pts):
    U.log("no-alloc uniform inputs")
    m, n, k = 600, 700, 304
    a_bits, b_bits = gen.operand_a(m, k, 9), gen.operand_b(k, n, 9)
    ref = oracle.gemm(a_bits, b_bits, m, n, k)
    a, b = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    for schedule in SCHEDULES:
        d = torch.full((m, n), float("nan"), dtype=torch.float32, device=U.DEV)
        _noalloc_c_abi(pts, pts.make_desc([(m, n, k)], schedule=_sched(pts, schedule)), [(a, b, d)])
        torch.cuda.synchronize()
        U.check_close(d, ref, k, f"no-alloc {schedule}")


def test_noalloc_allocates_nothing_and_rejects_oversize(pts):
    m = n = k = 256
    a = torch.zeros((m, k), dtype=torch.bfloat16, device=U.DEV)
    b = torch.zeros((n, k), dtype=torch.bfloat16, device=U.DEV)
    d = torch.empty((m, n), dtype=torch.float32, device=U.DEV)
    desc = pts.make_desc([(m, n, k)], schedule=pts.GEMM_SCHEDULE_DYNAMIC)
    _noalloc_c_abi(pts, desc, [(a, b, d)])     # the first call on the device looks up the scratch
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(200):
        _noalloc_c_abi(pts, desc, [(a, b, d)])
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) <= (2 << 20), f"free device memory moved by {free0 - free1} bytes over 200 calls"
    assert torch.all(d == 0)
    with pytest.raises(pts.GemmError) as ei:
        pts.gemm_run_noalloc(pts.make_desc([(8, 8, 8)] * (pts.GEMM_MAX_GROUPS + 1)), [(a, b, d)] * 65)
    assert ei.value.status == pts.GEMM_ERR_UNSUPPORTED and "at most" in str(ei.value)
