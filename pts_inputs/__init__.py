"""Seeded synthetic inputs for the persistent-tile bf16 GEMM.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark. It holds random-number generation only: a counter-based
SplitMix64 stream, the mapping of its outputs to uniform[-1, 1) values, and the
rounding of those generated values to bf16 bit patterns. It performs none of
the GEMM's arithmetic and imports neither the oracle nor the HIP library.

Generator (one fixed definition, used by every consumer):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): ``next()`` adds the odd constant
  ``GAMMA = 0x9E3779B97F4A7C15`` to a 64-bit state and returns ``mix64`` of the
  new state, where ``mix64`` is the variant-13 finalizer
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31``.
  Element ``i`` of a stream is therefore ``mix64(base + (i + 1) * GAMMA)``,
  which makes any slice regenerable without generating what precedes it.
* A stream is named by ``(seed, tensor_id)``:
  ``base = mix64((seed << 32) ^ tensor_id)`` with ``0 <= seed < 2**32``.
* uniform[-1, 1): ``u = (x >> 40) * 2**-24`` and ``v = 2u - 1``; ``v`` is exact
  in float32 and is rounded to bf16 with round-to-nearest-even.
* Integer-valued inputs for exact tests: ``((x >> 32) mod (2r + 1)) - r``.

Tensor ids used throughout: A = 1, B = 2, the grouped-problem M draw = 3,
the int16 copy source = 5, grouped problem g uses ``16 + 2g`` (A) and
``17 + 2g`` (B).
"""
from __future__ import annotations

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1

TENSOR_A = 1
TENSOR_B = 2
TENSOR_M_DRAW = 3
TENSOR_K_DRAW = 4
TENSOR_COPY_SRC = 5

_CHUNK = 1 << 18


def group_tensor_ids(g: int) -> tuple[int, int]:
    """Tensor ids of grouped problem ``g``'s A and B operands."""
    return 16 + 2 * g, 17 + 2 * g


def mix64_int(z: int) -> int:
    """SplitMix64 finalizer on a Python int (reference form, used for bases)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
    z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_MIX2)
        return z ^ (z >> np.uint64(31))


def stream_base(seed: int, tensor_id: int) -> int:
    if not (0 <= seed < (1 << 32)):
        raise ValueError("seed must be in [0, 2**32)")
    return mix64_int((seed << 32) ^ tensor_id)


def stream_u64(seed: int, tensor_id: int, count: int, start: int = 0) -> np.ndarray:
    """Elements ``start .. start+count-1`` of stream ``(seed, tensor_id)``."""
    base = np.uint64(stream_base(seed, tensor_id))
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64_np(base + idx * np.uint64(GAMMA))


def f32_to_bf16_bits_rne(v: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 bit patterns, nearest-even.

    Used only to turn generated float32 values into bf16 inputs.
    """
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    with np.errstate(over="ignore"):
        r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _uniform_chunk(seed: int, tensor_id: int, count: int, start: int) -> np.ndarray:
    x = stream_u64(seed, tensor_id, count, start)
    u24 = (x >> np.uint64(40)).astype(np.int64)
    v = ((2 * u24 - (1 << 24)).astype(np.float32)) * np.float32(2.0 ** -24)
    return f32_to_bf16_bits_rne(v)


def _threads() -> int:
    import os
    return max(1, min(16, os.cpu_count() or 1))


def uniform_bf16_bits(seed: int, tensor_id: int, count: int, start: int = 0,
                      out: np.ndarray | None = None) -> np.ndarray:
    """``count`` bf16 bit patterns of uniform[-1, 1) values, as uint16.

    Each element depends only on its own stream index, so large requests are
    split into chunks generated on several threads (numpy releases the GIL);
    the values do not depend on the split.
    """
    if out is None:
        out = np.empty(count, dtype=np.uint16)

    def fill(s):
        n = min(_CHUNK, count - s)
        out[s:s + n] = _uniform_chunk(seed, tensor_id, n, start + s)

    starts = range(0, count, _CHUNK)
    if count > 2 * _CHUNK and _threads() > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(_threads()) as pool:
            list(pool.map(fill, starts))
    else:
        for s in starts:
            fill(s)
    return out


def integer_bf16_bits(seed: int, tensor_id: int, count: int, radius: int = 4,
                      start: int = 0) -> np.ndarray:
    """Integers uniform in ``[-radius, radius]`` stored as bf16 bit patterns.

    Small integers are exact in bf16, so products and partial sums of such
    inputs are exact in float32 while their magnitude stays below 2**24.
    """
    if not (0 <= radius <= 128):
        raise ValueError("radius must be in [0, 128] to stay exact in bf16")
    x = stream_u64(seed, tensor_id, count, start)
    vals = ((x >> np.uint64(32)) % np.uint64(2 * radius + 1)).astype(np.int64) - radius
    return f32_to_bf16_bits_rne(vals.astype(np.float32))


def uniform_int16(seed: int, tensor_id: int, count: int) -> np.ndarray:
    """Raw int16 values (the low 16 bits of each stream element)."""
    out = np.empty(count, dtype=np.int16)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        out[s:s + n] = (stream_u64(seed, tensor_id, n, s) & np.uint64(0xFFFF)).astype(
            np.uint16).view(np.int16)
    return out


def matrix_row_major_bits(rows: int, cols: int, ld: int, seed: int, tensor_id: int,
                          kind: str = "uniform", radius: int = 4) -> np.ndarray:
    """A ``rows x ld`` uint16 buffer whose leading ``cols`` columns hold the stream.

    Element ``(r, c)`` with ``c < cols`` takes stream index ``r * cols + c``, so
    the values do not depend on the padding ``ld``. Padding columns are filled
    from stream ``tensor_id + 1000`` so that a reader that strays into them
    sees non-zero garbage.
    """
    if ld < cols:
        raise ValueError("ld must be >= cols")
    if kind == "uniform":
        vals = uniform_bf16_bits(seed, tensor_id, rows * cols)
    elif kind == "integer":
        vals = integer_bf16_bits(seed, tensor_id, rows * cols, radius)
    else:
        raise ValueError(kind)
    if ld == cols:
        return vals.reshape(rows, cols)
    buf = uniform_bf16_bits(seed, tensor_id + 1000, rows * ld).reshape(rows, ld)
    buf[:, :cols] = vals.reshape(rows, cols)
    return buf


def operand_a(m: int, k: int, seed: int = 0, lda: int | None = None,
              tensor_id: int = TENSOR_A, kind: str = "uniform", radius: int = 4) -> np.ndarray:
    """A (m x k, row-major): buffer ``m x lda``, ``A[i, kk] = buf[i, kk]``."""
    return matrix_row_major_bits(m, k, lda or k, seed, tensor_id, kind, radius)


def operand_b(k: int, n: int, seed: int = 0, ldb: int | None = None,
              tensor_id: int = TENSOR_B, kind: str = "uniform", radius: int = 4) -> np.ndarray:
    """B (k x n, column-major): buffer ``n x ldb``, ``B[kk, j] = buf[j, kk]``."""
    return matrix_row_major_bits(n, k, ldb or k, seed, tensor_id, kind, radius)


def grouped_m_draw(seed: int, groups: int = 64, step: int = 128, levels: int = 32) -> list[int]:
    """Problem heights ``M_g = step * (1 + floor(levels * u_g))``, u_g uniform[0, 1).

    With the defaults this draws each M_g uniformly from {128, 256, ..., 4096}.
    """
    x = stream_u64(seed, TENSOR_M_DRAW, groups)
    u24 = (x >> np.uint64(40)).astype(np.int64)
    return [int(step * (1 + (int(v) * levels >> 24))) for v in u24]


def grouped_k_draw(seed: int, groups: int = 64, step: int = 256, levels: int = 32) -> list[int]:
    """Per-problem depths ``K_g = step * (1 + floor(levels * u_g))`` from tensor id 4.

    With the defaults this draws each K_g uniformly from {256, 512, ..., 8192}:
    a grouped GEMM whose tiles cost in proportion to their problem's K.
    """
    x = stream_u64(seed, TENSOR_K_DRAW, groups)
    u24 = (x >> np.uint64(40)).astype(np.int64)
    return [int(step * (1 + (int(v) * levels >> 24))) for v in u24]


# ---------------------------------------------------------------------------
# Device-side generation (same stream, computed with torch int64 ops).
# ---------------------------------------------------------------------------

def _signed(c: int) -> int:
    return c - (1 << 64) if c >= (1 << 63) else c


def _torch_lsr(x, s: int):
    import torch
    return (x >> s) & torch.tensor((1 << (64 - s)) - 1, dtype=torch.int64, device=x.device)


def _torch_mix64(z):
    import torch
    m1 = torch.tensor(_signed(_MIX1), dtype=torch.int64, device=z.device)
    m2 = torch.tensor(_signed(_MIX2), dtype=torch.int64, device=z.device)
    z = (z ^ _torch_lsr(z, 30)) * m1
    z = (z ^ _torch_lsr(z, 27)) * m2
    return z ^ _torch_lsr(z, 31)


def uniform_bf16_torch(count: int, seed: int, tensor_id: int, device, start: int = 0,
                       chunk: int = 1 << 26):
    """Same values as :func:`uniform_bf16_bits`, generated with torch on ``device``.

    Returns a ``torch.bfloat16`` tensor of ``count`` elements. int64 arithmetic
    in torch wraps modulo 2**64, which is what the stream needs; the tests check
    this against the numpy definition.
    """
    import torch
    out = torch.empty(count, dtype=torch.int16, device=device)
    base = torch.tensor(_signed(stream_base(seed, tensor_id)), dtype=torch.int64, device=device)
    gamma = torch.tensor(_signed(GAMMA), dtype=torch.int64, device=device)
    for s in range(0, count, chunk):
        n = min(chunk, count - s)
        idx = torch.arange(start + s + 1, start + s + n + 1, dtype=torch.int64, device=device)
        x = _torch_mix64(base + idx * gamma)
        u24 = _torch_lsr(x, 40)
        v = (2 * u24 - (1 << 24)).to(torch.float32) * (2.0 ** -24)
        b = v.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
        r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
        out[s:s + n] = (r & 0xFFFF).to(torch.int32).to(torch.int16)
        del idx, x, u24, v, b, r
    return out.view(torch.bfloat16)
