"""Build the CPU oracle (oracle/liboracle.so) with gcc.

Test infrastructure: the oracle is a checker, never part of the product path.
Flags keep every fp32 operation a single IEEE operation: no FMA contraction,
no fast-math.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "bsfp_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


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
