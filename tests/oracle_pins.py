"""Pins for the GEMM oracle: checks that fix its result without trusting it.

Each check takes the oracle's entry points as arguments so that the same
checks run on the real oracle (``test_oracle_pins.py``) and on deliberately
broken copies of it (``test_oracle_mutants.py``), which must fail at least one.

What pins what:

* ``pin_integer_bruteforce`` -- integer-valued bf16 inputs make every product
  and partial sum exact, so the result must equal a Python big-integer sum
  built from the generator's integers (never decoded from bf16) for every
  small shape: pins the summation range, signs and both operand readings.
* ``pin_identity`` / ``pin_permutation`` -- B = I gives D = A exactly and a
  permutation matrix permutes the columns of A: pins the column-major
  reading of B and the row-major reading of A and D.
* ``pin_single_entry_probes`` -- A = e_i e_k^T against a B with all-distinct
  entries selects row k of B into row i of D: pins every index.
* ``pin_zero`` and ``pin_ones`` -- A = 0 gives 0; A = B = ones gives K exactly.
* ``pin_bf16_ties`` -- the two ties 3000 and 3016 (bf16 spacing 16 there)
  round to 3008 under ties-to-even, where truncation gives 2992 and
  round-half-away gives 3024.
* ``pin_numpy_matmul`` -- on random inputs the result agrees with numpy's
  float64 matmul of the decoded matrices (an independent library routine)
  within a few float64 rounding errors of sum |a||b|.
* ``pin_k_order`` -- products 1, 2^100, -2^100 (exact in bf16 and double):
  summed k ascending they give (1 + 2^100) - 2^100 = 0, summed in any order
  that adds the two large ones first they give 1: pins the summation order.
* ``pin_entries_integer`` -- the per-entry form on integer-valued inputs
  equals the same Python big-integer sums at every listed entry.
* ``pin_decode_vs_torch`` -- bf16 decoding agrees with torch's bf16 -> float64
  conversion on all 65536 patterns.
"""
from __future__ import annotations

import numpy as np

import pts_inputs as gen

BF16_ONE = 0x3F80


def _int_stream(seed, tid, count, radius=4):
    x = gen.stream_u64(seed, tid, count)
    return [int(v) - radius for v in ((x >> np.uint64(32)) % np.uint64(2 * radius + 1))]


def pin_integer_bruteforce(gemm, shapes, seed=7):
    for (m, n, k) in shapes:
        a = gen.operand_a(m, k, seed, kind="integer")
        b = gen.operand_b(k, n, seed, kind="integer")
        ia = _int_stream(seed, gen.TENSOR_A, m * k)
        ib = _int_stream(seed, gen.TENSOR_B, n * k)
        d = gemm(a, b, m, n, k)
        for i in range(m):
            for j in range(n):
                want = sum(ia[i * k + kk] * ib[j * k + kk] for kk in range(k))
                if d[i, j] != want:
                    raise AssertionError(f"integer brute force: shape {(m, n, k)} at {(i, j)}: "
                                         f"{d[i, j]} != {want}")


def pin_identity(gemm, decode, m=37, k=29, seed=3):
    a = gen.operand_a(m, k, seed)
    b = np.zeros((k, k), dtype=np.uint16)          # column-major: b[j, kk] = B[kk, j]
    np.fill_diagonal(b, BF16_ONE)
    d = gemm(a, b, m, k, k)
    if not np.array_equal(d, decode(a)):
        raise AssertionError("A . I != A")


def pin_permutation(gemm, decode, m=19, k=23, seed=5):
    a = gen.operand_a(m, k, seed)
    perm = np.random.default_rng(seed).permutation(k)
    b = np.zeros((k, k), dtype=np.uint16)          # B[perm[j], j] = 1  => D[:, j] = A[:, perm[j]]
    b[np.arange(k), perm] = BF16_ONE
    d = gemm(a, b, m, k, k)
    if not np.array_equal(d, decode(a)[:, perm]):
        raise AssertionError("A . P != A[:, perm]")


def pin_single_entry_probes(gemm, m=3, n=4, k=5):
    # B[kk, j] = 16 * kk + j + 1: distinct small integers, exact in bf16.
    bvals = np.array([[16 * kk + j + 1 for kk in range(k)] for j in range(n)], dtype=np.float32)
    b = gen.f32_to_bf16_bits_rne(bvals).reshape(n, k)
    for i in range(m):
        for kk in range(k):
            a = np.zeros((m, k), dtype=np.uint16)
            a[i, kk] = BF16_ONE
            d = gemm(a, b, m, n, k)
            want = np.zeros((m, n))
            want[i, :] = [16 * kk + j + 1 for j in range(n)]
            if not np.array_equal(d, want):
                raise AssertionError(f"probe A=e_{i} e_{kk}^T selects the wrong entries")


def pin_zero(gemm, m=33, n=17, k=40, seed=9):
    a = np.zeros((m, k), dtype=np.uint16)
    b = gen.operand_b(k, n, seed)
    if np.any(gemm(a, b, m, n, k) != 0):
        raise AssertionError("0 . B != 0")
    a = gen.operand_a(m, k, seed)
    b = np.full((n, k), 0x8000, dtype=np.uint16)    # -0.0
    if np.any(gemm(a, b, m, n, k) != 0):
        raise AssertionError("A . (-0) != 0")


def pin_ones(gemm, ks=(1, 2, 7, 64, 257, 3000, 3016)):
    for k in ks:
        a = np.full((2, k), BF16_ONE, dtype=np.uint16)
        b = np.full((3, k), BF16_ONE, dtype=np.uint16)
        d = gemm(a, b, 2, 3, k)
        if not np.all(d == k):
            raise AssertionError(f"ones: D != K for K={k}")


def pin_bf16_ties(gemm, round_bf16, decode):
    # bf16 spacing in [2048, 4096) is 16: 3000 = 2992 + 8 and 3016 = 3008 + 8 are
    # exact ties; ties-to-even keeps the even significand 3008 = 188 * 16 both times.
    for k, want in ((3000, 3008.0), (3016, 3008.0)):
        a = np.full((1, k), BF16_ONE, dtype=np.uint16)
        b = np.full((1, k), BF16_ONE, dtype=np.uint16)
        got = decode(round_bf16(gemm(a, b, 1, 1, k)))[0, 0]
        if got != want:
            raise AssertionError(f"RNE of {k} gave {got}, want {want}")


def pin_numpy_matmul(gemm, decode, m=67, n=45, k=301, seed=11):
    a = gen.operand_a(m, k, seed)
    b = gen.operand_b(k, n, seed)
    fa, fb = decode(a), decode(b)
    want = fa @ fb.T
    scale = np.abs(fa) @ np.abs(fb).T
    d = gemm(a, b, m, n, k)
    if np.any(np.abs(d - want) > 4 * k * 2.0 ** -53 * scale):
        raise AssertionError("disagrees with numpy float64 matmul")


def pin_k_order(gemm):
    big = 0x7180        # 2^100 in bf16
    a = np.array([[BF16_ONE, big, big | 0x8000]], dtype=np.uint16)   # 1, 2^100, -2^100
    b = np.full((2, 3), BF16_ONE, dtype=np.uint16)
    d = gemm(a, b, 1, 2, 3)
    if not np.all(d == 0.0):
        raise AssertionError(f"k order: got {d}, the ascending sum is 0")


def pin_entries_integer(gemm_entries, seed=13):
    for (m, n, k) in ((5, 4, 9), (3, 7, 1), (6, 6, 33)):
        a = gen.operand_a(m, k, seed, kind="integer")
        b = gen.operand_b(k, n, seed, kind="integer")
        ia = _int_stream(seed, gen.TENSOR_A, m * k)
        ib = _int_stream(seed, gen.TENSOR_B, n * k)
        rows = np.repeat(np.arange(m), n)
        cols = np.tile(np.arange(n), m)
        got = gemm_entries(a, b, k, rows, cols)
        for e, (i, j) in enumerate(zip(rows, cols)):
            want = sum(ia[i * k + kk] * ib[j * k + kk] for kk in range(k))
            if got[e] != want:
                raise AssertionError(f"entries: shape {(m, n, k)} at {(i, j)}: {got[e]} != {want}")


ALL_GEMM_PINS = ("integer_square", "integer", "identity", "permutation", "probes", "zero", "ones",
                 "ties", "numpy", "k_order", "entries_integer")


def run_gemm_pins(gemm, decode, round_bf16, on_result=None, gemm_entries=None):
    """Run every GEMM pin; return the names of those that failed.

    Square shapes run first: an index slip that swaps a dimension stays inside
    the buffers there, so it shows as a wrong value rather than a stray read.
    """
    shapes = [(m, n, k) for m in (1, 2, 5) for n in (1, 3, 4) for k in (1, 2, 6, 9)]
    checks = {
        "integer_square": lambda: pin_integer_bruteforce(gemm, [(s, s, s) for s in range(1, 7)]),
        "integer": lambda: pin_integer_bruteforce(gemm, shapes),
        "identity": lambda: pin_identity(gemm, decode),
        "permutation": lambda: pin_permutation(gemm, decode),
        "probes": lambda: pin_single_entry_probes(gemm),
        "zero": lambda: pin_zero(gemm),
        "ones": lambda: pin_ones(gemm),
        "ties": lambda: pin_bf16_ties(gemm, round_bf16, decode),
        "numpy": lambda: pin_numpy_matmul(gemm, decode),
        "k_order": lambda: pin_k_order(gemm),
    }
    if gemm_entries is not None:
        checks["entries_integer"] = lambda: pin_entries_integer(gemm_entries)
    failed = []
    for name, fn in checks.items():
        try:
            fn()
            ok = True
        except AssertionError:
            ok = False
            failed.append(name)
        if on_result is not None:
            on_result(name, ok)
    return failed
