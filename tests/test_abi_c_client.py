"""The boundary as a C interface: tests/abi_client.c, a plain C99 program
that includes only include/zs.h, is compiled with gcc (-std=c99 -pedantic
-Werror), linked against libzs.so and run on the host; the layout tables it
prints must equal the oracle's.  No GPU: only host calls."""

import os
import random
import shutil
import subprocess

import pytest

from oracle.layout import LayoutError, build_layout, build_tensor_layout
from tiles import n_tiles, tile_offsets
from synth import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_sharded_optimizer_shard_amd")
SRC = os.path.join(ROOT, "tests", "abi_client.c")


@pytest.fixture(scope="module")
def client(tmp_path_factory):
    if not os.path.exists(os.path.join(PKG, "libzs.so")):
        pytest.fail("libzs.so is not built (run __graft_entry__.build())")
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path_factory.mktemp("c") / "abi_client")
    subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra",
                    "-Werror", "-I", os.path.join(ROOT, "include"), SRC,
                    "-L", PKG, "-lzs", f"-Wl,-rpath,{PKG}", "-o", exe],
                   check=True, capture_output=True, text=True)
    return exe


def run(exe, mode, world, rank, cap, align, numels):
    p = subprocess.run([exe, mode, str(world), str(rank), str(cap),
                        str(align), *map(str, numels)],
                       check=True, capture_output=True, text=True)
    recs = {}
    for line in p.stdout.splitlines():
        k, *v = line.split()
        recs.setdefault(k, []).append(v)
    return recs


def expect(lay, world, rank, n_tensors, tensors):
    info = [str(lay.flat_numel), str(lay.shard_numel), str(len(lay.buckets)),
            str(len(lay.chunks)), str(n_tiles(lay)), str(world), str(rank)]
    out = {"info": [info],
           "tensor": [[str(t), str(o)] for t, o in
                      enumerate(lay.tensor_flat_off)],
           "bucket": [[str(x) for x in (b.flat_off, b.numel, b.slice_numel,
                                        b.shard_off, t0)]
                      for b, t0 in zip(lay.buckets, tile_offsets(lay))],
           "chunk": [[str(x) for x in (c.tensor_id, c.bucket_id,
                                       c.tensor_off, c.numel, c.shard_off)]
                     for c in lay.chunks]}
    if tensors:
        out["owner"] = [[str(t), str(r), str(o)] for t, (r, o) in
                        enumerate(zip(lay.owner, lay.owner_shard_off))]
    return {k: v for k, v in out.items() if v}


@pytest.mark.parametrize("seed", range(8))
def test_c_client_flat_layout(client, seed):
    rng = random.Random(7000 + seed)
    numels = [rng.choice([0, 1, 9, 128, 129, 4095, 50257, 70000])
              for _ in range(rng.randint(1, 10))]
    world = rng.choice([1, 2, 3, 8, 16])
    cap = rng.choice([0, 4096, 1 << 16, 25 << 20])
    align = rng.choice([16, 256])
    for rank in sorted({0, world - 1}):
        try:
            o = build_layout(numels, world, rank, cap, align)
        except LayoutError:
            got = run(client, "flat", world, rank, cap, align, numels)
            assert got["error"][0][0] == "-1"
            continue
        got = run(client, "flat", world, rank, cap, align, numels)
        assert got == expect(o, world, rank, len(numels), False)


@pytest.mark.parametrize("seed", range(6))
def test_c_client_whole_tensor_layout(client, seed):
    rng = random.Random(8000 + seed)
    numels = [rng.choice([0, 1, 7, 128, 1000, 4096, 70000])
              for _ in range(rng.randint(1, 12))]
    world = rng.choice([1, 2, 3, 5, 8])
    for rank in sorted({0, world - 1}):
        o = build_tensor_layout(numels, world, rank, 256)
        got = run(client, "tensors", world, rank, 0, 256, numels)
        assert got == expect(o, world, rank, len(numels), True)


def test_c_client_llama8b(client):
    w = wl.presets()["llama8b"]
    o = build_layout(w.numels, w.world, 3, 25 << 20, 256)
    got = run(client, "flat", w.world, 3, 25 << 20, 256, w.numels)
    assert got == expect(o, w.world, 3, len(w.numels), False)


def test_c_client_errors(client):
    got = run(client, "flat", 0, 0, 0, 256, [10])
    assert got["error"][0][0] == "-1"
    got = run(client, "flat", 2, 0, 0, 100, [10])          # align % 16
    assert got["error"][0][0] == "-1"
    got = run(client, "tensors", 1, 0, 0, 256, [(2 ** 21) * 8192])
    assert got["error"][0][0] == "-3"                      # launch limit
