"""CPU pins of the oracle (no GPU). See ``oracle_pins.py`` for what pins what."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import pts_inputs as gen
from tests import oracle_pins as pins


def test_gemm_pins_all_pass():
    assert pins.run_gemm_pins(oracle.gemm, oracle.bf16_decode, oracle.bf16_round,
                              gemm_entries=oracle.gemm_entries) == []


def test_bf16_decode_exhaustive_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros decode to signed zeros
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_bf16_round_vs_torch_on_float32_values():
    # torch's float32 -> bfloat16 conversion rounds to nearest, ties to even.
    rng = np.random.default_rng(0)
    patterns = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties and near-ties around every 16-bit boundary for a spread of exponents
    base = rng.integers(0, 1 << 16, size=20_000, dtype=np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base])
    allp = np.concatenate([patterns, ties]).view(np.float32)
    allp = allp[np.isfinite(allp)]
    ref = torch.from_numpy(allp.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.bf16_round(allp.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_round_special_values():
    r = oracle.bf16_round
    assert r(np.array([1 + 2.0 ** -8]))[0] == 0x3F80           # tie -> even (1.0)
    assert r(np.array([1 + 3 * 2.0 ** -8]))[0] == 0x3F82       # tie -> even (1 + 2^-6)
    assert r(np.array([3000.0]))[0] == r(np.array([3008.0]))[0]
    assert r(np.array([3016.0]))[0] == r(np.array([3008.0]))[0]
    assert r(np.array([3.4e38]))[0] == 0x7F80                  # past the midpoint to 2^128
    assert r(np.array([-(2 - 2.0 ** -7) * 2.0 ** 127]))[0] == 0xFF7F   # largest finite, negative
    assert r(np.array([(2 - 2.0 ** -8) * 2.0 ** 127]))[0] == 0x7F80    # midpoint to 2^128: tie to even (inf)
    assert r(np.array([2.0 ** -133]))[0] == 0x0001             # smallest subnormal
    assert r(np.array([2.0 ** -134]))[0] == 0x0000             # tie between 0 and 2^-133 -> 0
    assert r(np.array([3 * 2.0 ** -134]))[0] == 0x0002         # tie between 1 and 2 units -> 2
    assert r(np.array([-0.0]))[0] == 0x8000
    assert r(np.array([np.nan]))[0] & 0x7FC0 == 0x7FC0


def test_transpose_symmetry_bitwise():
    # (A.B)^T = B^T.A^T: B's column-major buffer is B^T row-major and A's row-major
    # buffer is A^T column-major, so swapping the buffers must give D^T bit for bit
    # (same products, same k order).
    m, n, k = 23, 31, 77
    a = gen.operand_a(m, k, 21)
    b = gen.operand_b(k, n, 21)
    d = oracle.gemm(a, b, m, n, k)
    dt = oracle.gemm(b, a, n, m, k)
    assert np.array_equal(d.T, dt)


def test_leading_dimension_padding_is_ignored():
    m, n, k = 17, 13, 40
    a_packed = gen.operand_a(m, k, 4)
    b_packed = gen.operand_b(k, n, 4)
    a_pad = gen.operand_a(m, k, 4, lda=k + 24)
    b_pad = gen.operand_b(k, n, 4, ldb=k + 8)
    assert np.array_equal(a_pad[:, :k], a_packed)
    d0 = oracle.gemm(a_packed, b_packed, m, n, k)
    d1 = oracle.gemm(a_pad, b_pad, m, n, k, lda=k + 24, ldb=k + 8)
    assert np.array_equal(d0, d1)


def test_entries_match_full_product_bitwise():
    m, n, k = 40, 50, 123
    a = gen.operand_a(m, k, 2)
    b = gen.operand_b(k, n, 2)
    d = oracle.gemm(a, b, m, n, k)
    rng = np.random.default_rng(1)
    rows = rng.integers(0, m, 300)
    cols = rng.integers(0, n, 300)
    assert np.array_equal(oracle.gemm_entries(a, b, k, rows, cols), d[rows, cols])


def test_thread_count_does_not_change_bits():
    m, n, k = 64, 48, 200
    a = gen.operand_a(m, k, 12)
    b = gen.operand_b(k, n, 12)
    assert np.array_equal(oracle.gemm(a, b, m, n, k, threads=1), oracle.gemm(a, b, m, n, k, threads=4))


def test_degenerate_shapes():
    a = gen.operand_a(5, 0, 1)
    b = gen.operand_b(0, 7, 1)
    d = oracle.gemm(np.zeros(0, np.uint16), np.zeros(0, np.uint16), 5, 7, 0)
    assert d.shape == (5, 7) and np.all(d == 0)          # K = 0: empty sum
    assert oracle.gemm(np.zeros(0, np.uint16), gen.operand_b(9, 4, 1), 0, 4, 9).shape == (0, 4)
    assert oracle.gemm(gen.operand_a(3, 9, 1), np.zeros(0, np.uint16), 3, 0, 9).shape == (3, 0)
    del a, b


def test_rejects_inconsistent_buffers():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros(10, np.uint16), np.zeros(10, np.uint16), 3, 3, 4)
    with pytest.raises(ValueError):
        oracle.gemm_entries(np.zeros(16, np.uint16), np.zeros(16, np.uint16), 4, [4], [0])


# ---------------------------------------------------------------------------
# Scheduler oracle
# ---------------------------------------------------------------------------

def _read_golden(path):
    table = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            w, tiles = line.split(":")
            table[int(w)] = [int(t) for t in tiles.split()]
    return table


def test_static_assignment_matches_printed_example(golden_dir):
    table = _read_golden(os.path.join(golden_dir, "static_grid_stride_12_tiles_4_workers.txt"))
    got = oracle.static_assignment(12, 4)
    assert {w: ts for w, ts in enumerate(got)} == table


@pytest.mark.parametrize("tiles,workers", [(1, 1), (5, 8), (16, 16), (560, 256), (1024, 256), (4097, 256)])
def test_static_assignment_covers_each_tile_once(tiles, workers):
    got = oracle.static_assignment(tiles, workers)
    flat = sorted(t for ts in got for t in ts)
    assert flat == list(range(tiles))
    # balanced to within one tile
    sizes = [len(ts) for ts in got]
    assert max(sizes) - min(sizes) <= 1


def test_dynamic_claim_checker_accepts_and_rejects():
    oracle.check_dynamic_claims([[0, 3, 4], [1, 2], [5]], 6)
    with pytest.raises(AssertionError):
        oracle.check_dynamic_claims([[0, 1], [1, 2]], 3)      # tile 1 twice
    with pytest.raises(AssertionError):
        oracle.check_dynamic_claims([[0], [2]], 3)            # tile 1 missing
    with pytest.raises(AssertionError):
        oracle.check_dynamic_claims([[2, 0], [1]], 3)         # not monotone


@pytest.mark.parametrize("shapes,bm,bn", [
    ([(256, 256)], 64, 64),
    ([(5000, 7000)], 256, 256),
    ([(129, 1), (1, 300), (256, 256), (0, 5)], 128, 128),
    ([(3, 3)], 256, 256),
])
def test_tile_coords_cover_every_element_once(shapes, bm, bn):
    tiles = oracle.tile_coords(shapes, bm, bn)
    offs = oracle.tile_offsets(shapes, bm, bn)
    assert len(tiles) == offs[-1]
    for g, (m, n) in enumerate(shapes):
        cover = np.zeros((m, n), dtype=np.int32)
        for (gg, r0, c0, vm, vn) in tiles:
            if gg == g:
                assert 0 < vm <= bm and 0 < vn <= bn
                cover[r0:r0 + vm, c0:c0 + vn] += 1
        assert np.all(cover == 1)
    assert sum(1 for t in tiles if t[0] == 1) == (offs[2] - offs[1] if len(shapes) > 1 else 0) or len(shapes) == 1


def test_ragged_config_tile_space():
    # 5000 x 7000 at 256 x 256: 20 x 28 = 560 tiles, last row 136 rows, last column 88 columns.
    tiles = oracle.tile_coords([(5000, 7000)], 256, 256)
    assert len(tiles) == 560
    assert tiles[-1][3:] == (136, 88)


def test_copy_oracle():
    src = gen.uniform_int16(0, gen.TENSOR_COPY_SRC, 1000)
    assert np.array_equal(oracle.copy_int16(src), src)
