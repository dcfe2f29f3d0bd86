"""Build the C oracle (``liboracle_gemm.so``) with gcc.

Test infrastructure: the oracle is compiled here and loaded only by the tests,
the smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_gemm.c")
LIB = os.path.join(HERE, "liboracle_gemm.so")

# -ffp-contract=off and no fast-math: each sum is evaluated exactly as written,
# k ascending, one rounding per addition (-O3 only vectorizes the i-k-j loop
# across independent output elements j).
CFLAGS = ["-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True, out: str = LIB, extra: list[str] | None = None) -> str:
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *(extra or []), SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
