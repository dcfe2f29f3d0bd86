"""C-ABI checks that need no GPU: exported symbols and host-side validation."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pts_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def binding():
    import persistent_tile_scheduling_amd as pts
    return pts


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gemm_plan_create", "gemm_run", "gemm_plan_destroy"):
        assert required in names
    assert len(names) >= 10


def test_library_exports_every_declared_symbol(binding):
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []


def test_binding_has_the_same_names(binding):
    for n in declared_functions():
        assert callable(getattr(binding, n)), n


def test_status_strings(binding):
    assert binding.gemm_status_string(0) == "success"
    assert "unsupported" in binding.gemm_status_string(2)
    assert binding.gemm_status_string(99) == "unknown status"


@pytest.mark.parametrize("kwargs,status,fragment", [
    (dict(layouts=(1, 1, 0)), 2, "layouts"),
    (dict(dtypes=(1, 0, 1)), 2, "bf16"),
    (dict(dtype_d=7), 2, "fp32 or bf16"),
    (dict(schedule=4), 1, "schedule"),
    (dict(schedule=-1), 1, "schedule"),
    (dict(schedule=3, num_workers=2), 1, "one workgroup per tile"),
    (dict(num_workers=-1), 1, "num_workers"),
    (dict(flags=0x80), 2, "flags"),
    (dict(flags=3), 2, "exclude each other"),
    (dict(flags=1, tile=(128, 128)), 2, "stage flags"),
    (dict(flags=2, tile=(256, 256, 0, 0, 0, 4)), 2, "stage flags"),
    (dict(flags=1, tile=(256, 256, 0, 0, 0, 8, 32)), 2, "stage flags"),
    (dict(flags=8), 1, "stall test flag"),
    (dict(tile=(96, 96)), 2, "not built"),
    (dict(tile=(-1, 256)), 1, "automatic tile"),
    (dict(tile=(-1, -1, 64)), 1, "automatic tile"),
    (dict(tile=(-1, -1, 0, 0, 0, 8)), 1, "automatic tile"),
    (dict(tile="auto", flags=1), 1, "automatic tile"),
])
def test_plan_create_rejects_bad_descriptors(binding, kwargs, status, fragment):
    with pytest.raises(binding.GemmError) as ei:
        binding.gemm_plan_create(binding.make_desc([(64, 64, 64)], **kwargs))
    assert ei.value.status == status
    assert fragment in str(ei.value)


@pytest.mark.parametrize("shape,fragment", [
    ((-1, 8, 8), "m, n, k"),
    ((8, 8, 12), "multiples of 8"),          # packed lda = 12
    ((8, 8, 16, 8, 16, 8), "leading dimension"),
    ((8, 8, 16, 16, 16, 4), "leading dimension"),
    ((8, 8, 16, 24, 20, 8), "multiples of 8"),
])
def test_plan_create_rejects_bad_shapes(binding, shape, fragment):
    with pytest.raises(binding.GemmError) as ei:
        binding.gemm_plan_create(binding.make_desc([shape]))
    assert ei.value.status == binding.GEMM_ERR_INVALID_VALUE
    assert fragment in str(ei.value)


def test_group_count_limits(binding):
    with pytest.raises(binding.GemmError) as ei:
        binding.gemm_plan_create(binding.make_desc([(8, 8, 8)] * (binding.GEMM_MAX_GROUPS + 1)))
    assert ei.value.status == binding.GEMM_ERR_UNSUPPORTED
    d = binding.make_desc([(8, 8, 8)])
    d.group_count = 0
    with pytest.raises(binding.GemmError):
        binding.gemm_plan_create(d)


def test_null_arguments(binding):
    lib = binding._lib
    out = ctypes.c_void_p(123)
    assert lib.gemm_plan_create(None, ctypes.byref(out)) == binding.GEMM_ERR_INVALID_VALUE
    assert out.value is None
    assert lib.gemm_plan_create(ctypes.byref(binding.make_desc([(8, 8, 8)])), None) == 1
    assert lib.gemm_run(None, None, None) == binding.GEMM_ERR_INVALID_VALUE
    assert lib.gemm_plan_destroy(None) == binding.GEMM_OK
    assert lib.gemm_plan_query(None, None, None, None) == binding.GEMM_ERR_INVALID_VALUE
    assert lib.pts_copy_int16(None, None, -1, 0, None) == binding.GEMM_ERR_INVALID_VALUE
    assert lib.pts_copy_int16(None, None, 0, 0, None) == binding.GEMM_OK     # empty copy is a no-op
    assert lib.pts_sched_probe(12, 0, 0, -1, 0, 0, None, None, 1, None, None, None) == 1
    assert lib.pts_stream_create_cu_masked(4, None) == binding.GEMM_ERR_INVALID_VALUE
    # the ceiling probe checks its sizes and pointers before any launch
    assert lib.pts_mfma_ceiling(None, None, None, 1, 2, None) == binding.GEMM_ERR_INVALID_VALUE
    assert lib.pts_mfma_ceiling(16, 16, 16, 1, 3, None) == binding.GEMM_ERR_INVALID_VALUE     # odd steps
    assert lib.pts_mfma_ceiling(16, 16, 16, -1, 2, None) == binding.GEMM_ERR_INVALID_VALUE
    assert lib.pts_mfma_ceiling(24, 16, 16, 1, 2, None) == binding.GEMM_ERR_INVALID_VALUE     # misaligned
    assert lib.pts_stream_destroy(None) == binding.GEMM_OK
    assert "NULL" in binding.gemm_last_error() or binding.gemm_last_error() != ""


def test_product_path_does_not_touch_the_oracle():
    # The HIP library's sources and the binding never mention the oracle package.
    pkg = os.path.join(ROOT, "persistent_tile_scheduling_amd")
    for d, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(d, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle_gemm" not in text, f


def test_header_constants_match_the_binding(binding):
    import re
    text = open(os.path.join(ROOT, "include", "pts_gemm.h")).read()
    defines = dict(re.findall(r"#define ((?:GEMM|PTS)_[A-Z_]+) (\d+)", text))
    assert defines, "no numeric constants found in the header"
    for name, value in defines.items():
        assert getattr(binding, name) == int(value), name
    negative = dict(re.findall(r"#define (GEMM_[A-Z_]+) \((-\d+)\)", text))
    assert "GEMM_TILE_AUTO" in negative
    for name, value in negative.items():
        assert getattr(binding, name) == int(value), name
    enums = dict(re.findall(r"(GEMM_SCHEDULE_[A-Z_]+) = (\d+)", text))
    for name, value in enums.items():
        assert getattr(binding, name) == int(value), name


@pytest.mark.parametrize("shape,fragment", [
    ((256, 8, 8, 1 << 23, 8, 8), "32-bit"),              # a tile's rows of A span more than 2^31 bytes
    ((8, 256, 8, 8, 1 << 23, 256), "32-bit"),            # same for the columns of B
    ((1 << 30, 1 << 30, 8), "output tiles"),             # tile count beyond the claim encoding
    ((1 << 31, 8, 8), "m, n, k"),
])
def test_plan_create_rejects_sizes_beyond_the_limits(binding, shape, fragment):
    with pytest.raises(binding.GemmError) as ei:
        binding.gemm_plan_create(binding.make_desc([shape]))
    assert ei.value.status in (binding.GEMM_ERR_INVALID_VALUE, binding.GEMM_ERR_UNSUPPORTED)
    assert fragment in str(ei.value)


def test_tile_strings_other_than_auto_are_rejected(binding):
    with pytest.raises(ValueError):
        binding.make_desc([(64, 64, 64)], tile="largest")
    d = binding.make_desc([(64, 64, 64)], tile="auto")
    assert (d.tile_m, d.tile_n) == (binding.GEMM_TILE_AUTO, binding.GEMM_TILE_AUTO)


def test_gemm_convenience_checks_dtypes_before_anything_else(binding):
    import torch
    a = torch.zeros((8, 8), dtype=torch.float32)
    b = torch.zeros((8, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.gemm(a, b)
    with pytest.raises(ValueError):
        binding.gemm(b, b[0])
