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
    "drops_last_k": ("kk < k; ++kk)\n                acc +=", "kk < k - 1; ++kk)\n                acc +="),
    "skips_first_k": ("for (int64_t kk = 0; kk < k; ++kk)\n                acc +=",
                      "for (int64_t kk = 1; kk < k; ++kk)\n                acc +="),
    "subtracts": ("acc += oracle_bf16_decode(a[i * lda + kk])", "acc -= oracle_bf16_decode(a[i * lda + kk])"),
    "b_row_major": ("oracle_bf16_decode(b[j * ldb + kk]);\n            d[",
                    "oracle_bf16_decode(b[kk * ldb + j]);\n            d["),
    "a_uses_col": ("acc += oracle_bf16_decode(a[i * lda + kk]) * oracle_bf16_decode(b[j * ldb + kk]);\n            d[",
                   "acc += oracle_bf16_decode(a[j * lda + kk]) * oracle_bf16_decode(b[j * ldb + kk]);\n            d["),
    "d_transposed": ("d[i * ldd + j] = acc;", "d[j * ldd + i] = acc;"),
    "decode_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "round_half_away": ("rint(ldexp(x, -q))", "round(ldexp(x, -q))"),
    "round_truncates": ("rint(ldexp(x, -q))", "trunc(ldexp(x, -q))"),
    "accumulates_float": ("double acc = 0.0;\n            for (int64_t kk = 0; kk < k; ++kk)\n                acc +=",
                          "float acc = 0.0f;\n            for (int64_t kk = 0; kk < k; ++kk)\n                acc += (float)"),
}

_CHILD = r"""
import json, sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins as pins
lib = oracle.OracleLib({lib!r})
def report(name, ok):
    print(json.dumps([name, ok]), flush=True)
pins.run_gemm_pins(lib.gemm, lib.bf16_decode, lib.bf16_round, on_result=report)
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
