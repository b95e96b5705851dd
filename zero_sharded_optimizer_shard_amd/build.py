"""Build libzs.so (the C-ABI library of include/zs.h) for gfx950, in-tree.

Flags that matter for the arithmetic: -ffp-contract=off (one rounding per
fp32 operation, no fused multiply-add), hipcc's default correctly rounded
fp32 divide and square root, IEEE denormals (no flush), and packed fp32
instructions disabled.
"""

import hashlib
import json
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libzs.so")
# sha256 prefix of every kernel's machine code in LIB, written by build()
KERNELS = os.path.join(PKG, "libzs.kernels.json")
LLVM = "/opt/rocm/llvm/bin"

SOURCES = [os.path.join(CSRC, "zs_layout.cpp"),
           os.path.join(CSRC, "zs_step.hip"),
           os.path.join(CSRC, "zs_gather.hip"),
           os.path.join(CSRC, "zs_accum.hip"),
           os.path.join(CSRC, "zs_stream.cpp"),
           os.path.join(CSRC, "zs_prefetch.cpp"),
           os.path.join(CSRC, "zs_ckpt.cpp")]

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
    with open(KERNELS, "w") as f:
        json.dump(kernel_digests(LIB), f, indent=0, sort_keys=True)
    return LIB


def _tool(name, *args) -> str:
    return subprocess.run([os.path.join(LLVM, name), *args], check=True,
                          capture_output=True, text=True).stdout


def kernel_digests(lib: str) -> dict:
    """{mangled kernel name: sha256 prefix of its machine code} for the
    gfx950 code object embedded in `lib` (a library built here).  Identical
    bytes mean an identical kernel, whatever else changed in the sources;
    measurements tied to one kernel (its HBM counters) stay valid while its
    digest does."""
    out = {}
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        _tool("llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", lib,
              os.path.join(d, "rest.so"))
        # one offload bundle per source file with device code
        blob = open(fat, "rb").read()
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        starts = [m.start() for m in re.finditer(re.escape(magic), blob)]
        for i, a in enumerate(starts):
            part = os.path.join(d, f"b{i}.bin")
            co = os.path.join(d, f"b{i}.elf")
            end = starts[i + 1] if i + 1 < len(starts) else len(blob)
            with open(part, "wb") as f:
                f.write(blob[a:end])
            _tool("clang-offload-bundler", "--unbundle", "--type=o",
                  f"--input={part}", f"--output={co}",
                  "--targets=hipv4-amdgcn-amd-amdhsa--gfx950")
            out.update(_elf_kernel_digests(co))
    return out


def _elf_kernel_digests(co: str) -> dict:
    data = open(co, "rb").read()
    text = None
    for line in _tool("llvm-readelf", "-S", "-W", co).splitlines():
        m = re.search(r"\]\s+\.text\s+PROGBITS\s+([0-9a-f]+)\s+"
                      r"([0-9a-f]+)", line)
        if m:
            text = (int(m.group(1), 16), int(m.group(2), 16))
    out = {}
    if text is None:
        return out
    for line in _tool("llvm-readelf", "-s", "-W", co).splitlines():
        f = line.split()
        if len(f) >= 8 and f[3] == "FUNC" and f[2] != "0":
            off = int(f[1], 16) - text[0] + text[1]
            code = data[off:off + int(f[2])]
            out[f[7]] = hashlib.sha256(code).hexdigest()[:16]
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
