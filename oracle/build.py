"""Compile the CPU oracle (plain C, gcc) into ``oracle/libw4oracle.so``.

Test infrastructure: the library built here is only ever loaded by the tests,
the smoke check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w4_oracle.c")
OUT = os.path.join(HERE, "libw4oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
          "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
