"""Build the C step oracle (test infrastructure) into oracle/libzs_oracle.so.

Plain C, -O2, no FMA contraction, no fast-math, no flush-to-zero, so that
every fp32 statement of the oracle is one IEEE operation rounded to nearest.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zs_oracle.c")
LIB = os.path.join(HERE, "libzs_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", SRC, "-o", LIB + ".tmp",
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
