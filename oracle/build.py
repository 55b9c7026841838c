"""Builds the CPU oracle shared library (test infrastructure, never the product path).

The flags matter: no fast-math and no floating-point contraction, so that every
fp32 operation of the routing arithmetic rounds exactly as written in the C source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O3", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
