"""Build the CPU oracle (plain C, gcc + OpenMP) into oracle/liboracle_w4a8.so.

Test infrastructure only.  The flags keep every fp32 operation a single IEEE-754
round-to-nearest-even operation: no FMA contraction, no fast-math, SSE arithmetic.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w4a8_oracle.c")
LIB = os.path.join(HERE, "liboracle_w4a8.so")

CFLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra",
          "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
