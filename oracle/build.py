"""Build the CPU oracle (test infrastructure) as oracle/liboracle.so.

The oracle is plain C built with gcc at -O2 with no fast-math and no FMA
contraction, so that every binary32 operation in it rounds exactly once.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qcp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
