"""Build the synthetic-input libraries: libsynth_cpu.so (gcc, OpenMP) and
libsynth_dev.so (hipcc, gfx950)."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> None:
    cpu = os.path.join(HERE, "libsynth_cpu.so")
    _run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
          "-Wextra", os.path.join(HERE, "gen.c"), "-o", cpu + ".tmp"],
         verbose)
    os.replace(cpu + ".tmp", cpu)
    dev = os.path.join(HERE, "libsynth_dev.so")
    _run(["hipcc", *HIP_FLAGS, os.path.join(HERE, "gen.hip"),
          "-o", dev + ".tmp"], verbose)
    os.replace(dev + ".tmp", dev)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
