"""Compile the fp64 oracle (plain C, gcc, OpenMP) into oracle/liboracle.so.

Test infrastructure: the oracle is only ever loaded by the tests, the smoke
check and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # No -march=native: the library is built here and also runs on other hosts.
    # -ffp-contract=off keeps every sum a plain IEEE add (products are exact anyway).
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-Wall", "-Wextra",
           os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
