"""Compile the C oracle into oracle/liboracle.so (test infrastructure only).

The oracle is a plain CPU program; building it is part of building the
repository's checkers, not of the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rowstats_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# No fast-math and no FMA contraction: every fp32 and fp64 operation is the
# plain IEEE operation written in the source.
CFLAGS = ["-O2", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-fopenmp",
          "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
