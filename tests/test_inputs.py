"""CPU tests of the seeded input generator (no GPU)."""
from __future__ import annotations

import numpy as np
import torch

import pts_inputs as gen


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 1234567 (Vigna's reference splitmix64.c): the first
    # outputs are mix64(1234567 + GAMMA), mix64(1234567 + 2*GAMMA), ...
    state = 1234567
    outs = []
    for _ in range(3):
        state = (state + gen.GAMMA) & ((1 << 64) - 1)
        outs.append(gen.mix64_int(state))
    assert outs == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_stream_is_counter_based():
    full = gen.stream_u64(0, 1, 1000)
    part = gen.stream_u64(0, 1, 100, start=500)
    assert np.array_equal(full[500:600], part)
    base = gen.stream_base(0, 1)
    i = 37
    assert int(full[i]) == gen.mix64_int(base + (i + 1) * gen.GAMMA)


def test_streams_differ_by_seed_and_tensor():
    assert not np.array_equal(gen.stream_u64(0, 1, 64), gen.stream_u64(0, 2, 64))
    assert not np.array_equal(gen.stream_u64(0, 1, 64), gen.stream_u64(1, 1, 64))


def test_uniform_values_in_range_and_bf16_exact():
    bits = gen.uniform_bf16_bits(0, 1, 200_000)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert vals.min() >= -1.0 and vals.max() <= 1.0
    assert abs(vals.mean()) < 0.01 and abs(vals.var() - 1.0 / 3.0) < 0.01


def test_uniform_rounding_matches_torch():
    x = gen.stream_u64(0, 1, 50_000)
    v = ((2 * (x >> np.uint64(40)).astype(np.int64) - (1 << 24)).astype(np.float32)) * np.float32(2.0 ** -24)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.uniform_bf16_bits(0, 1, 50_000), ref)


def test_chunked_generation_matches_unchunked():
    n = (1 << 22) + 12345
    a = gen.uniform_bf16_bits(3, 9, n)
    assert np.array_equal(a[(1 << 22) - 5:(1 << 22) + 5], gen.uniform_bf16_bits(3, 9, 10, start=(1 << 22) - 5))


def test_torch_generator_matches_numpy_on_cpu():
    n = 100_003
    t = gen.uniform_bf16_torch(n, 0, 1, "cpu", chunk=1 << 15)
    assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), gen.uniform_bf16_bits(0, 1, n))
    t2 = gen.uniform_bf16_torch(1000, 5, 17, "cpu", start=777)
    assert np.array_equal(t2.view(torch.int16).numpy().view(np.uint16), gen.uniform_bf16_bits(5, 17, 1000, start=777))


def test_integer_inputs():
    bits = gen.integer_bf16_bits(0, 1, 10_000, radius=4)
    vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert set(np.unique(vals)) == set(range(-4, 5))


def test_grouped_m_draw():
    ms = gen.grouped_m_draw(0)
    assert len(ms) == 64
    assert all(m % 128 == 0 and 128 <= m <= 4096 for m in ms)
    assert gen.grouped_m_draw(0) == ms
    assert len(set(ms)) > 16


def test_grouped_k_draw():
    ks = gen.grouped_k_draw(0)
    assert len(ks) == 64
    assert all(k % 256 == 0 and 256 <= k <= 8192 for k in ks)
    assert gen.grouped_k_draw(0) == ks
    assert len(set(ks)) > 16
    assert ks != gen.grouped_m_draw(0, step=256)   # its own tensor id, not the M draw's


def test_operand_layouts_and_padding():
    a = gen.operand_a(4, 6, 0, lda=16)
    assert a.shape == (4, 16)
    assert np.array_equal(a[:, :6], gen.operand_a(4, 6, 0))
    b = gen.operand_b(6, 3, 0)
    assert b.shape == (3, 6)          # column-major K x N is stored as N rows of K
