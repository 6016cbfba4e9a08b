"""Builds the oracle's C library (oracle/libssd_oracle.so) with gcc.

TEST INFRASTRUCTURE ONLY. Plain -O2 without fast-math, so the floating-point
evaluation order is exactly the one written in ssd_oracle.c.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "libssd_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
