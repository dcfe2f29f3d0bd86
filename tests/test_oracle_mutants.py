"""Plant mistakes in copies of the oracle (on the CPU) and check the pins catch them.

Each mutant is the oracle's C source with one plausible slip applied -- a
dropped term, a wrong start, a sign, a transposed operand, the wrong rounding
-- built into a temporary library and run against the pins in a child
process. Every mutant must fail at least one pin, which
shows the pins constrain each part of the oracle.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    # the full product (i, k, j loop over the row-major copy of B)
    "drops_last_k": ("for (int64_t kk = 0; kk < k; ++kk) {\n            const double aik",
                     "for (int64_t kk = 0; kk < k - 1; ++kk) {\n            const double aik"),
    "skips_first_k": ("for (int64_t kk = 0; kk < k; ++kk) {\n            const double aik",
                      "for (int64_t kk = 1; kk < k; ++kk) {\n            const double aik"),
    "subtracts": ("drow[j] += aik * decode(brow[j]);", "drow[j] -= aik * decode(brow[j]);"),
    "b_row_major": ("bt[kk * n + j] = b[j * ldb + kk];", "bt[kk * n + j] = b[kk * ldb + j];"),
    "a_uses_col": ("const double aik = decode(a[i * lda + kk]);", "const double aik = decode(a[kk * lda + i]);"),
    "b_copy_transposed_twice": ("const uint16_t *brow = bt + kk * n;\n            for (int64_t j = 0; j < n; ++j)\n"
                                "                drow[j] += aik * decode(brow[j]);",
                                "const uint16_t *brow = bt + kk;\n            for (int64_t j = 0; j < n; ++j)\n"
                                "                drow[j] += aik * decode(brow[j * k]);"),
    "d_transposed": ("double *drow = d + i * ldd;", "double *drow = d + i;"),
    "d_not_cleared": ("            drow[j] = 0.0;\n", "            drow[j] += 0.0;\n"),
    "decode_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "round_half_away": ("rint(ldexp(x, -q))", "round(ldexp(x, -q))"),
    "round_truncates": ("rint(ldexp(x, -q))", "trunc(ldexp(x, -q))"),
    "accumulates_float": ("drow[j] += aik * decode(brow[j]);", "drow[j] = (float)(drow[j] + aik * decode(brow[j]));"),
    # the per-entry form
    "entries_drop_last_k": ("for (int64_t kk = 0; kk < k; ++kk)\n            acc +=",
                            "for (int64_t kk = 0; kk < k - 1; ++kk)\n            acc +="),
    "k_descending": ("for (int64_t kk = 0; kk < k; ++kk) {\n            const double aik = decode(a[i * lda + kk]);\n"
                     "            const uint16_t *brow = bt + kk * n;",
                     "for (int64_t k2 = 0; k2 < k; ++k2) {\n            const int64_t kk = k - 1 - k2;\n"
                     "            const double aik = decode(a[i * lda + kk]);\n"
                     "            const uint16_t *brow = bt + kk * n;"),
    "entries_b_row_major": ("acc += decode(a[i * lda + kk]) * decode(b[j * ldb + kk]);",
                            "acc += decode(a[i * lda + kk]) * decode(b[kk * ldb + j]);"),
}

_CHILD = r"""
import json, sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins as pins
lib = oracle.OracleLib({lib!r})
def report(name, ok):
    print(json.dumps([name, ok]), flush=True)
pins.run_gemm_pins(lib.gemm, lib.bf16_decode, lib.bf16_round, on_result=report, gemm_entries=lib.gemm_entries)
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found in the oracle source"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new, 1))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", *obuild.CFLAGS, str(mutant_src), "-o", str(lib), "-lm"], check=True,
                   capture_output=True)
    proc = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=str(lib))],
                          capture_output=True, text=True, timeout=300,
                          env={**os.environ, "OMP_NUM_THREADS": "2"})
    results = [json.loads(line) for line in proc.stdout.splitlines() if line.startswith("[")]
    failed = [pin for pin, ok in results if not ok]
    # A pin must fail before anything else happens; a crash afterwards (a stray
    # read on a later, non-square shape) does not count as the catch.
    assert failed, f"mutant {name} passed every pin it reached (exit status {proc.returncode})"
