"""Build the HIP library (``_lib/libpts_gemm.so``) for gfx950 with hipcc.

The library has no torch dependency; the Python binding loads it with ctypes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIB_DIR, "libpts_gemm.so")
SOURCES = [os.path.join(CSRC, "pts_gemm.hip")]
ARCH = os.environ.get("PTS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed fp32 instructions are kept out of the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The scheduler's claim is one lane's atomic whose result is read a tile
    # later. The atomic optimizer would rewrite it into a wave-wide form that
    # reads the result at once, i.e. waits for the round trip on the spot.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    warnings = [ln for ln in (res.stdout + res.stderr).splitlines()
                if "warning" in ln and "packed-fp32-ops" not in ln]
    if warnings and verbose:
        sys.stderr.write("\n".join(warnings) + "\n")
    os.replace(tmp, out)
    return out


def sources_newer_than(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    for d, _, files in os.walk(CSRC):
        for f in files:
            if os.path.getmtime(os.path.join(d, f)) > t:
                return True
    return os.path.getmtime(os.path.join(INCLUDE, "pts_gemm.h")) > t


if __name__ == "__main__":
    print(build(verbose=True))
