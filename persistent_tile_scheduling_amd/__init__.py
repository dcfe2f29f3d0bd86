"""Python binding of the persistent-tile-scheduled bf16 GEMM library.

Argument marshalling only: every step of the GEMM runs in the HIP kernels of
``_lib/libpts_gemm.so`` (built from ``csrc/`` by ``build.py``). The functions
carry the C ABI's names (``include/pts_gemm.h``); ``Plan`` and ``gemm`` are
small conveniences over them that take torch tensors for device memory.

There is no fallback: importing this package raises if the HIP library has
not been built, and every call raises ``GemmError`` on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so that the library binds to torch's HIP runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libpts_gemm.so")

GEMM_OK = 0
GEMM_ERR_INVALID_VALUE = 1
GEMM_ERR_UNSUPPORTED = 2
GEMM_ERR_OUT_OF_MEMORY = 3
GEMM_ERR_HIP = 4
GEMM_ERR_TIMEOUT = 5

GEMM_DTYPE_BF16 = 0
GEMM_DTYPE_F32 = 1
GEMM_ROW_MAJOR = 0
GEMM_COL_MAJOR = 1
GEMM_SCHEDULE_STATIC = 0
GEMM_SCHEDULE_DYNAMIC = 1
GEMM_SCHEDULE_DYNAMIC_XCD = 2
GEMM_SCHEDULE_NONPERSISTENT = 3
GEMM_SCHED_COUNTER_BYTES = 36864
GEMM_MAX_GROUPS = 64
GEMM_NOALLOC_SCRATCH_BYTES = 40960
GEMM_TILE_AUTO = -1
GEMM_FLAG_NONE = 0
GEMM_FLAG_STAGE_FLAGS_FUSED = 1
GEMM_FLAG_STAGE_FLAGS_MERGED = 2
GEMM_FLAG_PROBLEM_ORDER_AS_GIVEN = 4
GEMM_FLAG_DEBUG_STAGE_FLAG_STALL = 8
GEMM_FLAG_CLAIM_AFTER_TILE = 16
PTS_MFMA_CEILING_FRAG_BYTES = 196608

TILE_TRACE_BYTES = 56
WORKER_TRACE_BYTES = 32


class GemmShape(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldd", ctypes.c_int64)]


class GemmDesc(ctypes.Structure):
    _fields_ = [("group_count", ctypes.c_int32), ("shapes", ctypes.POINTER(GemmShape)),
                ("layout_a", ctypes.c_int32), ("layout_b", ctypes.c_int32), ("layout_d", ctypes.c_int32),
                ("dtype_a", ctypes.c_int32), ("dtype_b", ctypes.c_int32), ("dtype_acc", ctypes.c_int32),
                ("dtype_d", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("stages", ctypes.c_int32), ("load_path", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("mfma", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("num_workers", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class GemmOperands(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("d", ctypes.c_void_p)]


class GemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                          "(run persistent_tile_scheduling_amd/build.py or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sig = {
        "gemm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "gemm_last_error": (ctypes.c_char_p, []),
        "gemm_plan_create": (ctypes.c_int, [ctypes.POINTER(GemmDesc), ctypes.POINTER(P)]),
        "gemm_run": (ctypes.c_int, [P, ctypes.POINTER(GemmOperands), P]),
        "gemm_plan_destroy": (ctypes.c_int, [P]),
        "gemm_plan_query": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]),
        "gemm_plan_query_kernel": (ctypes.c_int, [P] + [ctypes.POINTER(ctypes.c_int32)] * 6),
        "gemm_plan_set_trace": (ctypes.c_int, [P, P, ctypes.c_size_t]),
        "gemm_plan_read_counters": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_uint32)]),
        "gemm_plan_preset_claims": (ctypes.c_int, [P, ctypes.c_uint32]),
        "gemm_run_noalloc": (ctypes.c_int, [ctypes.POINTER(GemmDesc), ctypes.POINTER(GemmOperands), P]),
        "pts_copy_int16": (ctypes.c_int, [P, P, ctypes.c_int64, ctypes.c_int32, P]),
        "pts_stream_create_cu_masked": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(P)]),
        "pts_stream_destroy": (ctypes.c_int, [P]),
        "pts_sched_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int64, ctypes.c_int64, P, P, ctypes.c_int32, P, P, P]),
        "pts_mfma_ceiling": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int) -> None:
    if status != GEMM_OK:
        raise GemmError(status, _lib.gemm_last_error().decode() or gemm_status_string(status))


def _stream_handle(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.data_ptr()
    return int(t)


# ---------------------------------------------------------------------------
# C ABI, same names
# ---------------------------------------------------------------------------

def gemm_status_string(status: int) -> str:
    return _lib.gemm_status_string(status).decode()


def gemm_last_error() -> str:
    return _lib.gemm_last_error().decode()


def make_desc(shapes, dtype_d: int = GEMM_DTYPE_F32, tile=(0, 0, 0, 0, 0, 0, 0), schedule: int = GEMM_SCHEDULE_STATIC,
              num_workers: int = 0, flags: int = GEMM_FLAG_NONE, layouts=(GEMM_ROW_MAJOR, GEMM_COL_MAJOR,
                                                                           GEMM_ROW_MAJOR),
              dtypes=(GEMM_DTYPE_BF16, GEMM_DTYPE_BF16, GEMM_DTYPE_F32)):
    """Build a ``gemm_desc``. ``shapes`` is a list of (m, n, k[, lda, ldb, ldd]);
    ``tile`` is (tile_m, tile_n[, tile_k, stages, load_path, waves, mfma]) with 0 for defaults,
    or "auto" for tile_m = tile_n = GEMM_TILE_AUTO (chosen by size)."""
    if isinstance(tile, str):
        if tile != "auto":
            raise ValueError(f"tile must be a tuple or 'auto', not {tile!r}")
        tile = (GEMM_TILE_AUTO, GEMM_TILE_AUTO)
    arr = (GemmShape * max(1, len(shapes)))()
    for i, s in enumerate(shapes):
        s = tuple(s) + (0,) * (6 - len(s))
        arr[i] = GemmShape(*[int(v) for v in s])
    tile = tuple(tile) + (0,) * (7 - len(tile))
    d = GemmDesc(len(shapes), ctypes.cast(arr, ctypes.POINTER(GemmShape)), layouts[0], layouts[1], layouts[2],
                 dtypes[0], dtypes[1], dtypes[2], dtype_d, tile[0], tile[1], tile[2], tile[3], tile[4], tile[5],
                 tile[6], schedule, num_workers, flags)
    d._shapes_keepalive = arr
    return d


def gemm_plan_create(desc: GemmDesc) -> int:
    out = ctypes.c_void_p()
    _check(_lib.gemm_plan_create(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def gemm_run(plan: int, operands, stream=None) -> None:
    """``operands``: list of (a, b, d) device pointers or tensors, one per problem."""
    arr = (GemmOperands * max(1, len(operands)))()
    for i, (a, b, d) in enumerate(operands):
        arr[i] = GemmOperands(_ptr(a), _ptr(b), _ptr(d))
    _check(_lib.gemm_run(ctypes.c_void_p(plan), arr, ctypes.c_void_p(_stream_handle(stream))))


def gemm_run_noalloc(desc: GemmDesc, operands, stream=None) -> None:
    """gemm_run without a plan: validates ``desc`` and runs it using the
    library's per-GPU scratch array (no device allocation)."""
    arr = (GemmOperands * max(1, len(operands)))()
    for i, (a, b, d) in enumerate(operands):
        arr[i] = GemmOperands(_ptr(a), _ptr(b), _ptr(d))
    _check(_lib.gemm_run_noalloc(ctypes.byref(desc), arr, ctypes.c_void_p(_stream_handle(stream))))


def gemm_plan_destroy(plan: int | None) -> None:
    _check(_lib.gemm_plan_destroy(ctypes.c_void_p(plan)))


def gemm_plan_query(plan: int) -> tuple[int, int, int]:
    t, w, l = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.gemm_plan_query(ctypes.c_void_p(plan), ctypes.byref(t), ctypes.byref(w), ctypes.byref(l)))
    return t.value, w.value, l.value


def gemm_plan_query_kernel(plan: int) -> dict:
    """The plan's kernel: tile_m, tile_n, tile_k, stages, waves, mfma."""
    vals = [ctypes.c_int32() for _ in range(6)]
    _check(_lib.gemm_plan_query_kernel(ctypes.c_void_p(plan), *[ctypes.byref(v) for v in vals]))
    return dict(zip(("tile_m", "tile_n", "tile_k", "stages", "waves", "mfma"), (v.value for v in vals)))


def gemm_plan_set_trace(plan: int, device_buf, nbytes: int) -> None:
    _check(_lib.gemm_plan_set_trace(ctypes.c_void_p(plan), ctypes.c_void_p(_ptr(device_buf)), nbytes))


def gemm_plan_read_counters(plan: int) -> list[int]:
    out = (ctypes.c_uint32 * 5)()
    _check(_lib.gemm_plan_read_counters(ctypes.c_void_p(plan), out))
    return list(out)


def gemm_plan_preset_claims(plan: int, value: int) -> None:
    """Test only: the dynamic schedules' claim counters start the next run at ``value``."""
    _check(_lib.gemm_plan_preset_claims(ctypes.c_void_p(plan), value))


def pts_copy_int16(src, dst, n: int, num_blocks: int = 0, stream=None) -> None:
    _check(_lib.pts_copy_int16(ctypes.c_void_p(_ptr(src)), ctypes.c_void_p(_ptr(dst)), n, num_blocks,
                               ctypes.c_void_p(_stream_handle(stream))))


def pts_stream_create_cu_masked(cu_count: int) -> int:
    """A raw stream handle whose kernels run only on the first cu_count CUs."""
    out = ctypes.c_void_p()
    _check(_lib.pts_stream_create_cu_masked(cu_count, ctypes.byref(out)))
    return int(out.value)


def pts_stream_destroy(stream: int) -> None:
    _check(_lib.pts_stream_destroy(ctypes.c_void_p(stream)))


def pts_sched_probe(num_tiles: int, num_workers: int, schedule: int, gate_worker: int, work_ns: int,
                    spin_limit: int, out_tiles, out_counts, max_per_worker: int, counters, out_status,
                    stream=None) -> None:
    _check(_lib.pts_sched_probe(num_tiles, num_workers, schedule, gate_worker, work_ns, spin_limit,
                                ctypes.c_void_p(_ptr(out_tiles)), ctypes.c_void_p(_ptr(out_counts)),
                                max_per_worker, ctypes.c_void_p(_ptr(counters)),
                                ctypes.c_void_p(_ptr(out_status)), ctypes.c_void_p(_stream_handle(stream))))


def pts_mfma_ceiling(frags, out, stamps, num_blocks: int, steps: int, stream=None) -> None:
    _check(_lib.pts_mfma_ceiling(ctypes.c_void_p(_ptr(frags)), ctypes.c_void_p(_ptr(out)),
                                 ctypes.c_void_p(_ptr(stamps)), num_blocks, steps,
                                 ctypes.c_void_p(_stream_handle(stream))))


# ---------------------------------------------------------------------------
# Conveniences over the C ABI
# ---------------------------------------------------------------------------

class Plan:
    """Owns one ``gemm_plan``. ``shapes``: list of (m, n, k[, lda, ldb, ldd]);
    ``tile``: (tile_m, tile_n[, tile_k, stages, load_path, waves, mfma]), 0 = default,
    or "auto" (the library picks the tile edge from the sizes)."""

    def __init__(self, shapes, out_dtype=torch.float32, tile=(0, 0), schedule: str | int = "static",
                 num_workers: int = 0, flags: int = GEMM_FLAG_NONE):
        if isinstance(schedule, str):
            schedule = {"static": GEMM_SCHEDULE_STATIC, "dynamic": GEMM_SCHEDULE_DYNAMIC,
                        "dynamic_xcd": GEMM_SCHEDULE_DYNAMIC_XCD,
                        "nonpersistent": GEMM_SCHEDULE_NONPERSISTENT}[schedule]
        dtype_d = {torch.float32: GEMM_DTYPE_F32, torch.bfloat16: GEMM_DTYPE_BF16}[out_dtype]
        self.shapes = [tuple(s) for s in shapes]
        self.out_dtype = out_dtype
        self.schedule = schedule
        self.desc = make_desc(self.shapes, dtype_d, tile, schedule, num_workers, flags)
        self.handle = gemm_plan_create(self.desc)
        self.num_tiles, self.num_workers, self.lds_bytes = gemm_plan_query(self.handle)
        self.kernel = gemm_plan_query_kernel(self.handle)

    def run(self, operands, stream=None) -> None:
        gemm_run(self.handle, operands, stream)

    def counters(self) -> list[int]:
        return gemm_plan_read_counters(self.handle)

    def preset_claims(self, value: int) -> None:
        gemm_plan_preset_claims(self.handle, value)

    def trace_bytes(self) -> int:
        return TILE_TRACE_BYTES * self.num_tiles + WORKER_TRACE_BYTES * self.num_workers

    def set_trace(self, buf) -> None:
        gemm_plan_set_trace(self.handle, buf, 0 if buf is None else buf.numel() * buf.element_size())

    def close(self) -> None:
        if self.handle:
            gemm_plan_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_trace(buf: torch.Tensor, num_tiles: int, num_workers: int):
    """Split a trace buffer (any dtype, on any device) into numpy record arrays."""
    import numpy as np
    raw = buf.detach().cpu().contiguous().view(torch.uint8).numpy()
    tile_dt = np.dtype([("tile", "<i4"), ("claim", "<i4"), ("worker", "<i4"), ("seq", "<i4"), ("group", "<i4"),
                        ("row0", "<i4"), ("col0", "<i4"), ("xcc_id", "<u4"), ("cycles", "<u4"), ("pad", "<u4"),
                        ("t_start", "<u8"), ("t_end", "<u8")])
    worker_dt = np.dtype([("t_start", "<u8"), ("t_end", "<u8"), ("tiles", "<i4"), ("worker", "<i4"),
                          ("hw_id", "<u4"), ("xcc_id", "<u4")])
    nt = TILE_TRACE_BYTES * num_tiles
    tiles = raw[:nt].view(tile_dt)
    workers = raw[nt:nt + WORKER_TRACE_BYTES * num_workers].view(worker_dt)
    return tiles, workers


def gemm(a: torch.Tensor, b: torch.Tensor, out_dtype=torch.float32, schedule="static", tile="auto",
         num_workers: int = 0, out: torch.Tensor | None = None, k: int | None = None) -> torch.Tensor:
    """D = A . B for a bf16 A (m x k, row-major) and B given as its transpose
    (n x k, row-major: B's columns are the rows of ``b``).

    ``a`` and ``b`` may be row slices or column slices of larger tensors
    (``x[:, :k]``): their leading dimensions are taken from ``stride(0)``, which
    must be a multiple of 8 elements, ``stride(1)`` must be 1 and the first
    element 16-byte aligned. ``k``
    defaults to ``a.shape[1]``. ``out`` (fp32 or bf16, m x n, ``stride(1) == 1``)
    is written in place when given and must not share memory with ``a`` or ``b``
    (not checked). Every tensor must be on the current GPU.
    Anything else raises ``ValueError``. Builds a one-shot plan; the tile
    defaults to the library's choice for the sizes ("auto").
    """
    for name, t in (("a", a), ("b", b)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 2:
            raise ValueError(f"{name} must be a 2-D bfloat16 tensor")
    m, ka = a.shape
    n, kb = b.shape
    kk = ka if k is None else int(k)
    if kk < 0 or kk > ka or kk > kb:
        raise ValueError(f"k = {kk} exceeds the operands' widths ({ka}, {kb})")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=a.device)
    if out.dtype not in (torch.float32, torch.bfloat16) or out.dim() != 2 or tuple(out.shape) != (m, n):
        raise ValueError(f"out must be a 2-D fp32 or bf16 tensor of shape ({m}, {n})")
    dev = torch.device("cuda", torch.cuda.current_device())
    for name, t in (("a", a), ("b", b), ("out", out)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, not on the current device {dev}")
        if t.numel() and t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{name} must have unit stride along its rows (stride(1) == 1)")
    lda = a.stride(0) if m > 1 else 8 * ((kk + 7) // 8)
    ldb = b.stride(0) if n > 1 else 8 * ((kk + 7) // 8)
    ldd = out.stride(0) if m > 1 else n
    if lda % 8 or ldb % 8:
        raise ValueError(f"row strides of a and b ({lda}, {ldb}) must be multiples of 8 elements")
    if kk and (a.data_ptr() % 16 or b.data_ptr() % 16):
        raise ValueError("a and b must start 16-byte aligned (a column slice must start at a multiple of 8)")
    if ldd < n:
        raise ValueError(f"out's row stride {ldd} is below n = {n}")
    with Plan([(m, n, kk, lda, ldb, ldd)], out.dtype, tile, schedule, num_workers) as p:
        p.run([(a, b, out)])
    return out
