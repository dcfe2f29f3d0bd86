"""GPU tests of the binding's ``gemm()`` convenience: leading dimensions come
from the tensors' strides, so sliced and padded operands give the oracle's
result, and every layout it cannot pass to the library is refused."""
from __future__ import annotations

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


def test_gemm_on_column_slices_and_padded_out(pts):
    m, n, k = 300, 200, 136
    lda, ldb, ldd = 160, 144, 232
    a_bits = gen.operand_a(m, k, 31, lda=lda, kind="integer")
    b_bits = gen.operand_b(k, n, 31, ldb=ldb, kind="integer")
    ref = oracle.gemm(a_bits, b_bits, m, n, k, lda=lda, ldb=ldb)
    a_full, b_full = U.bits_to_device(a_bits), U.bits_to_device(b_bits)
    a, b = a_full[:, :k], b_full[:, :k]                 # views: stride(0) = lda, ldb
    assert a.stride(0) == lda and b.stride(0) == ldb
    for out_dtype in (torch.float32, torch.bfloat16):
        backing = torch.full((m + 2, ldd), 9.0, dtype=out_dtype, device=U.DEV)
        out = backing[:m, :n]
        for schedule in ("static", "dynamic_xcd"):
            res = pts.gemm(a, b, schedule=schedule, out=out)
            torch.cuda.synchronize()
            assert res.data_ptr() == out.data_ptr()
            U.check_exact(out.contiguous(), ref, f"gemm() {out_dtype} {schedule}")
            assert torch.all(backing[:m, n:] == 9.0) and torch.all(backing[m:] == 9.0)
    # k below the operands' width: only the first k columns take part
    k2 = 64
    ref2 = oracle.gemm(a_bits, b_bits, m, n, k2, lda=lda, ldb=ldb)
    d2 = pts.gemm(a_full, b_full, k=k2)
    torch.cuda.synchronize()
    U.check_exact(d2, ref2, "gemm() k < width")


def test_gemm_refuses_what_it_cannot_pass(pts):
    a = torch.zeros((64, 64), dtype=torch.bfloat16, device=U.DEV)
    b = torch.zeros((64, 64), dtype=torch.bfloat16, device=U.DEV)
    with pytest.raises(ValueError):
        pts.gemm(a.float(), b)                              # fp32 operand read as bf16 bits
    with pytest.raises(ValueError):
        pts.gemm(a, b.t())                                  # stride(1) != 1
    with pytest.raises(ValueError):
        pts.gemm(a, torch.zeros((64, 72), dtype=torch.bfloat16, device=U.DEV)[:, 3:67])  # misaligned start
    with pytest.raises(ValueError):
        pts.gemm(torch.zeros((64, 68), dtype=torch.bfloat16, device=U.DEV)[:, :64], b)    # lda 68
    with pytest.raises(ValueError):
        pts.gemm(a, b, out=torch.zeros((64, 64), dtype=torch.float32, device=U.DEV).t())
    with pytest.raises(ValueError):
        pts.gemm(a, b, out=torch.zeros((64, 63), dtype=torch.float32, device=U.DEV))
    with pytest.raises(ValueError):
        pts.gemm(a, b.cpu())
    with pytest.raises(ValueError):
        pts.gemm(a, b, k=65)
