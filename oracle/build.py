"""Compile the CPU oracle (oracle.c) into liboracle.so with gcc.

Test infrastructure: the oracle is built so that tests, the smoke check and the benchmark's
CPU baseline can call it; the product library never links or loads it.

Flags: -O2 without fast-math, -ffp-contract=off so that no multiply-add is fused and the
double-precision sums keep their written order, OpenMP over independent vocabulary rows.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-fopenmp", "-Wall", "-Wextra"]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
