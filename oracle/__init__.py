"""CPU oracle for the persistent-tile bf16 GEMM.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers. The HIP library and its
Python binding never import this package, and this package imports nothing
from them.

Three oracles, each written from the pages' definitions:

* ``gemm`` / ``gemm_entries`` / ``grouped_gemm`` -- the matrix product D = A.B
  in double (C, ``oracle_gemm.c``), following the GEMM mainloop of the CUTLASS
  Task Scheduling page "Pipeline Groups", section "Overview" (smem_a and smem_b
  consumed together into the accumulator, the accumulator stored to D).
* ``static_assignment`` / ``tile_coords`` -- the persistent scheduler: which
  output tiles exist and which worker a static grid-stride schedule gives each
  one ("Advanced scheduling: Cluster Launch Control", section "Limits of the
  static persistent scheduler": with 12 tiles and 4 workers, worker w takes
  tiles w, w+4, w+8), and the exactly-once property of dynamic claiming (same
  section: each coordinate is processed exactly once, either by its own CTA or
  by the worker that took it over).
* ``copy_int16`` -- the grid-stride copy of the CUTLASS Task Scheduling page
  "Schedules", section "Domains": every in-range index i gets dst[i] = src[i].
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        x = x.view(np.uint16) if x.dtype.itemsize == 2 else x.astype(np.uint16)
    return x


def _check_operands(m, n, k, a, lda, b, ldb):
    if min(m, n, k) < 0:
        raise ValueError("negative dimension")
    if lda < k or ldb < k:
        raise ValueError("leading dimension smaller than K")
    if m and k and a.size < (m - 1) * lda + k:
        raise ValueError("A buffer too small")
    if n and k and b.size < (n - 1) * ldb + k:
        raise ValueError("B buffer too small")


class OracleLib:
    """The C oracle loaded from one shared-library file."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_bf16_decode_array.argtypes = [_u16p, _f64p, ctypes.c_int64]
        lib.oracle_bf16_round_array.argtypes = [_f64p, _u16p, ctypes.c_int64]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    _u16p, ctypes.c_int64, _u16p, ctypes.c_int64,
                                    _f64p, ctypes.c_int64, ctypes.c_int]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm_entries.argtypes = [ctypes.c_int64, _u16p, ctypes.c_int64,
                                            _u16p, ctypes.c_int64, ctypes.c_int64,
                                            _i64p, _i64p, _f64p, ctypes.c_int]
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def bf16_decode(self, bits) -> np.ndarray:
        """bf16 bit patterns -> float64, exactly."""
        b = _u16(bits)
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_bf16_decode_array(b.ctypes.data_as(_u16p), out.ctypes.data_as(_f64p), b.size)
        return out

    def bf16_round(self, x) -> np.ndarray:
        """float64 -> bf16 bit patterns, round to nearest, ties to even."""
        v = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.oracle_bf16_round_array(v.ctypes.data_as(_f64p), out.ctypes.data_as(_u16p), v.size)
        return out

    def gemm(self, a_bits, b_bits, m: int, n: int, k: int, lda: int | None = None,
             ldb: int | None = None, threads: int = 0) -> np.ndarray:
        """D (m x n float64) = A . B with A row-major (lda) and B column-major (ldb).

        ``a_bits`` is a uint16 buffer with ``A[i, kk] = a[i * lda + kk]``;
        ``b_bits`` is a uint16 buffer with ``B[kk, j] = b[j * ldb + kk]``.
        """
        lda = k if lda is None else lda
        ldb = k if ldb is None else ldb
        a = _u16(a_bits).reshape(-1)
        b = _u16(b_bits).reshape(-1)
        _check_operands(m, n, k, a, lda, b, ldb)
        # NaN-filled: an element the C loop failed to clear or write shows up
        d = np.full((m, n), np.nan, dtype=np.float64)
        if m and n:
            if self.lib.oracle_gemm(m, n, k, a.ctypes.data_as(_u16p), lda, b.ctypes.data_as(_u16p), ldb,
                                    d.ctypes.data_as(_f64p), n, threads) != 0:
                raise MemoryError(f"oracle: no memory for the row-major copy of B ({k} x {n})")
        return d

    def gemm_entries(self, a_bits, b_bits, k: int, rows, cols, lda: int | None = None,
                     ldb: int | None = None, threads: int = 0) -> np.ndarray:
        """D[rows[e], cols[e]] for each listed entry, by the same definition."""
        lda = k if lda is None else lda
        ldb = k if ldb is None else ldb
        a = _u16(a_bits).reshape(-1)
        b = _u16(b_bits).reshape(-1)
        r = np.ascontiguousarray(rows, dtype=np.int64)
        c = np.ascontiguousarray(cols, dtype=np.int64)
        if r.shape != c.shape:
            raise ValueError("rows and cols differ in shape")
        if r.size and (r.min() < 0 or c.min() < 0):
            raise ValueError("negative index")
        if r.size and k and ((r.max() * lda + k > a.size) or (c.max() * ldb + k > b.size)):
            raise ValueError("entry outside the operand buffers")
        out = np.zeros(r.shape, dtype=np.float64)
        if r.size:
            self.lib.oracle_gemm_entries(k, a.ctypes.data_as(_u16p), lda, b.ctypes.data_as(_u16p), ldb,
                                         r.size, r.ctypes.data_as(_i64p), c.ctypes.data_as(_i64p),
                                         out.ctypes.data_as(_f64p), threads)
        return out


_default: OracleLib | None = None


def _lib() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build(force=True)
        _default = OracleLib(_build.LIB)
    return _default


def max_threads() -> int:
    return _lib().max_threads()


def bf16_decode(bits) -> np.ndarray:
    return _lib().bf16_decode(bits)


def bf16_round(x) -> np.ndarray:
    return _lib().bf16_round(x)


def gemm(a_bits, b_bits, m, n, k, lda=None, ldb=None, threads=0) -> np.ndarray:
    return _lib().gemm(a_bits, b_bits, m, n, k, lda, ldb, threads)


def gemm_entries(a_bits, b_bits, k, rows, cols, lda=None, ldb=None, threads=0) -> np.ndarray:
    return _lib().gemm_entries(a_bits, b_bits, k, rows, cols, lda, ldb, threads)


gemm.__doc__ = OracleLib.gemm.__doc__
gemm_entries.__doc__ = OracleLib.gemm_entries.__doc__
bf16_decode.__doc__ = OracleLib.bf16_decode.__doc__
bf16_round.__doc__ = OracleLib.bf16_round.__doc__


def grouped_gemm(problems, threads: int = 0) -> list[np.ndarray]:
    """Independent products, one per problem ``(a_bits, b_bits, m, n, k, lda, ldb)``."""
    return [gemm(a, b, m, n, k, lda, ldb, threads) for (a, b, m, n, k, lda, ldb) in problems]


# ---------------------------------------------------------------------------
# Scheduler
# ---------------------------------------------------------------------------

def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def tile_coords(shapes, bm: int, bn: int) -> list[tuple[int, int, int, int, int]]:
    """Every output tile of a (grouped) problem, in plain order.

    ``shapes`` is a list of ``(m, n)``. Tiles are numbered problem by problem;
    problem g owns the index range ``offsets[g] .. offsets[g+1]-1`` with
    ``offsets[g+1] = offsets[g] + ceil(m_g/bm) * ceil(n_g/bn)``, the offsets-array
    construction of the "Schedules" page, section "Dynamic Domain". Inside a
    problem the tiles are listed row-major. Each tile is
    ``(g, row0, col0, valid_rows, valid_cols)``.
    """
    out = []
    for g, (m, n) in enumerate(shapes):
        for tm in range(ceil_div(m, bm)):
            for tn in range(ceil_div(n, bn)):
                r0, c0 = tm * bm, tn * bn
                out.append((g, r0, c0, min(bm, m - r0), min(bn, n - c0)))
    return out


def tile_offsets(shapes, bm: int, bn: int) -> list[int]:
    offs = [0]
    for (m, n) in shapes:
        offs.append(offs[-1] + ceil_div(m, bm) * ceil_div(n, bn))
    return offs


def static_assignment(num_tiles: int, num_workers: int) -> list[list[int]]:
    """Static grid-stride schedule: worker w takes tiles w, w+P, w+2P, ... < T."""
    if num_workers <= 0:
        raise ValueError("need at least one worker")
    return [list(range(w, num_tiles, num_workers)) for w in range(num_workers)]


def check_dynamic_claims(per_worker: list[list[int]], num_tiles: int) -> None:
    """Raise AssertionError unless the claims cover every tile exactly once.

    Each worker's claims come from one monotone counter, so they must also be
    strictly increasing within a worker.
    """
    seen = sorted(t for ts in per_worker for t in ts)
    if seen != list(range(num_tiles)):
        raise AssertionError("tiles not covered exactly once")
    for ts in per_worker:
        if any(x >= y for x, y in zip(ts, ts[1:])):
            raise AssertionError("a worker's claims are not increasing")


# ---------------------------------------------------------------------------
# Copy
# ---------------------------------------------------------------------------

def copy_int16(src) -> np.ndarray:
    """dst[i] = src[i] for every in-range i."""
    return np.array(src, dtype=np.int16, copy=True)
