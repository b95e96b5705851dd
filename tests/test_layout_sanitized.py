"""The host half of the library under AddressSanitizer and UBSan: the
layout builder (csrc/zs_layout.cpp, plain C++) and tests/abi_client.c are
built with g++/gcc and -fsanitize=address,undefined, then run over random
lists, the workload lists and the error paths with halt_on_error and leak
checking on; each run must exit cleanly with the oracle's tables.  Host
code only: no GPU, no HIP."""

import os
import random
import shutil
import subprocess

import pytest

from oracle.layout import LayoutError, build_layout, build_tensor_layout
from synth import workloads as wl
from test_abi_c_client import expect

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "zero_sharded_optimizer_shard_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer",
       "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ,
           ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if gxx is None or gcc is None:
        pytest.skip("g++/gcc not found")
    d = tmp_path_factory.mktemp("san")
    lib = str(d / "libzs.so")
    exe = str(d / "abi_client")
    subprocess.run([gxx, "-std=c++17", *SAN, "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "zs_layout.cpp"), "-o", lib],
                   check=True, capture_output=True, text=True)
    subprocess.run([gcc, "-std=c99", *SAN, "-I",
                    os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_client.c"),
                    "-L", str(d), "-lzs", f"-Wl,-rpath,{d}", "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def run(exe, mode, world, rank, cap, align, numels):
    p = subprocess.run([exe, mode, str(world), str(rank), str(cap),
                        str(align), *map(str, numels)],
                       capture_output=True, text=True, env=ENV)
    assert p.returncode == 0 and "runtime error" not in p.stderr and \
        "Sanitizer" not in p.stderr, p.stderr[-3000:]
    recs = {}
    for line in p.stdout.splitlines():
        k, *v = line.split()
        recs.setdefault(k, []).append(v)
    return recs


@pytest.mark.parametrize("seed", range(6))
def test_sanitized_random_layouts(client, seed):
    rng = random.Random(9000 + seed)
    for _ in range(6):
        numels = [rng.choice([0, 1, 7, 128, 129, 4095, 50257, 70000])
                  for _ in range(rng.randint(0, 14))]
        world = rng.choice([1, 2, 3, 5, 8, 16, 64])
        rank = rng.randrange(world)
        cap = rng.choice([0, -1, 4096, 1 << 16, 25 << 20])
        align = rng.choice([16, 48, 256, 4096])
        try:
            o = build_layout(numels, world, rank, cap, align)
        except LayoutError:
            assert run(client, "flat", world, rank, cap, align,
                       numels)["error"][0][0] == "-1"
        else:
            got = run(client, "flat", world, rank, cap, align, numels)
            assert got == expect(o, world, rank, len(numels), False)
        o = build_tensor_layout(numels, world, rank, 256)
        got = run(client, "tensors", world, rank, 0, 256, numels)
        assert got == expect(o, world, rank, len(numels), True)


@pytest.mark.parametrize("name", ["tiny", "gpt2", "llama8b", "dense7b",
                                  "llama70b"])
def test_sanitized_workload_layouts(client, name):
    w = wl.presets()[name]
    r = w.world - 1
    o = build_layout(w.numels, w.world, r, 25 << 20, 256)
    got = run(client, "flat", w.world, r, 25 << 20, 256, w.numels)
    assert got == expect(o, w.world, r, len(w.numels), False)
    o = build_tensor_layout(w.numels, w.world, r, 256)
    got = run(client, "tensors", w.world, r, 0, 256, w.numels)
    assert got == expect(o, w.world, r, len(w.numels), True)


def test_sanitized_error_paths(client):
    big = 2 ** 62
    cases = [("flat", 0, 0, 0, 256, [5], "-1"),        # world < 1
             ("flat", 4, 4, 0, 256, [5], "-1"),        # rank >= world
             ("flat", 2, 0, 0, 100, [5], "-1"),        # align % 16
             ("flat", 2, 0, 0, 256, [-3], "-1"),       # negative numel
             ("flat", 8, 0, 1000, 256, [5], "-1"),     # cap below W*align
             ("flat", 2, 0, 0, 256, [big, big], "-3"),  # int64 overflow
             ("tensors", 2, 0, 0, 256, [big, big], "-3"),
             ("tensors", 1, 0, 0, 256, [2 ** 21 * 8192], "-3")]  # launch
    for mode, world, rank, cap, align, numels, code in cases:
        got = run(client, mode, world, rank, cap, align, numels)
        assert got["error"][0][0] == code, (mode, world, numels, got)
