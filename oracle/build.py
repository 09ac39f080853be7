"""Compile the fp64 CPU oracle (attn_oracle.c) into liboracle.so with gcc.

Test infrastructure only: the oracle is the checker for the GPU library and is
never linked into it.  No fast-math and no FMA contraction, so every sum is the
plain sequential double-precision sum the source spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O3", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
