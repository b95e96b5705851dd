"""Build libzs.so (the C-ABI library of include/zs.h) for gfx950, in-tree.

Flags that matter for the arithmetic: -ffp-contract=off (one rounding per
fp32 operation, no fused multiply-add), hipcc's default correctly rounded
fp32 divide and square root, IEEE denormals (no flush), and packed fp32
instructions disabled.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libzs.so")

SOURCES = [os.path.join(CSRC, "zs_layout.cpp"),
           os.path.join(CSRC, "zs_step.hip"),
           os.path.join(CSRC, "zs_gather.hip"),
           os.path.join(CSRC, "zs_accum.hip")]

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-fno-gpu-flush-denormals-to-zero",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False, extra=()) -> str:
    cmd = ["hipcc", *HIP_FLAGS, *extra, "-shared", *SOURCES,
           "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    msg = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
