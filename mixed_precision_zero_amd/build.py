"""Build libz1.so for gfx950 in-tree with hipcc.

Flags that matter for the results:
  -ffp-contract=off      no fused multiply-add is formed from separate
                         multiplies and adds, so every binary64 operation of
                         the AdamW update rounds where the definition rounds
  (no fast-math)         IEEE division and square root, denormals kept
  -target-feature -packed-fp32-ops
                         no packed two-lane fp32 instructions are generated
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libz1.so")
SOURCES = [os.path.join(CSRC, "z1_api.hip"), os.path.join(CSRC, "z1_kernels.hip"),
           os.path.join(CSRC, "z1_probe.hip")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


def command(out: str = LIB) -> list:
    return [HIPCC, *FLAGS, "-o", out, *SOURCES]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)   # never leave a half-written library behind
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
