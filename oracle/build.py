"""Compile the oracle (plain C, binary64) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is the CPU statement of what the GPU library
computes; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "skinny_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    # -O2 without -ffast-math: IEEE binary64 semantics, no contraction of
    # multiply-add pairs, so every rounding is the one the source states.
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
