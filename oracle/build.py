"""Build the CPU oracle (test infrastructure) into oracle/libstep5_oracle.so.

Plain C, gcc, no contraction of multiply-adds and no fast-math, so that every
float operation in the oracle is the single IEEE operation written in the
source.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libstep5_oracle.so")
SRC = os.path.join(HERE, "step5_oracle.c")

CFLAGS = ["-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
