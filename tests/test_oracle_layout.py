"""Pins of the layout oracle (oracle/layout.py) against rules it does not
share code with: per-element brute force, the plain reduce-scatter chunking
of a single flat buffer, and the partition / alignment / cap invariants."""

import random

import numpy as np
import pytest

from oracle.layout import LayoutError, build_layout, shard_flat_index
from synth import workloads as wl


def brute_force(numels, world, rank, cap_bytes, align_bytes):
    """Per-element construction from the definitions, no interval maths."""
    A = align_bytes // 2
    owner = []                       # flat position -> (tensor, offset) | None
    for t, n in enumerate(numels):
        while len(owner) % A:
            owner.append(None)
        owner.extend((t, k) for k in range(n))
    L = len(owner)
    unit = world * A
    if cap_bytes <= 0:
        full = max(-(-L // unit) * unit, unit)
    else:
        full = (cap_bytes // 2) // unit * unit
    # walk the flat buffer, opening a bucket every `full` elements
    buckets = []
    pos = 0
    while pos < L:
        size = min(full, -(-(L - pos) // unit) * unit)
        buckets.append((pos, size))
        pos += size
    owner.extend([None] * (pos - L))
    # the rank's shard, element by element, in bucket order
    shard = []
    for b, (off, size) in enumerate(buckets):
        sl = size // world
        for p in range(off + rank * sl, off + (rank + 1) * sl):
            shard.append((b, owner[p]))
    # maximal runs
    chunks = []
    for i, (b, o) in enumerate(shard):
        if o is None:
            continue
        t, k = o
        if chunks:
            ct, cb, coff, cn, cs = chunks[-1]
            if ct == t and cb == b and coff + cn == k and cs + cn == i:
                chunks[-1] = (ct, cb, coff, cn + 1, cs)
                continue
        chunks.append((t, b, k, 1, i))
    return pos, len(shard), buckets, chunks


def as_tuples(lay):
    return [(c.tensor_id, c.bucket_id, c.tensor_off, c.numel, c.shard_off)
            for c in lay.chunks]


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_random_lists(seed):
    rng = random.Random(seed)
    numels = [rng.choice([0, 1, 7, 8, 127, 128, 129, 300, 1000, 2047, 5000])
              for _ in range(rng.randint(1, 9))]
    world = rng.choice([1, 2, 3, 4, 5, 8])
    align = rng.choice([16, 32, 256])
    cap = rng.choice([0, -1, 1 << 12, 3000 * 2, 5 << 10, 1 << 20])
    if 0 < cap and (cap // 2) < world * align // 2:
        cap = 1 << 14
    for rank in range(world):
        lay = build_layout(numels, world, rank, cap, align)
        flat, shard, buckets, chunks = brute_force(numels, world, rank, cap,
                                                   align)
        assert lay.flat_numel == flat
        assert lay.shard_numel == shard
        assert [(b.flat_off, b.numel) for b in lay.buckets] == buckets
        assert as_tuples(lay) == chunks


@pytest.mark.parametrize("world", [1, 2, 3, 5, 8])
def test_single_bucket_is_plain_reduce_scatter_chunking(world):
    """With no bucketing the rank's shard is the r-th of W equal chunks of
    the flat buffer, as the sketch's single reduce_scatter_tensor gives."""
    numels = [1000, 129, 7, 4096, 33]
    for rank in range(world):
        lay = build_layout(numels, world, rank, 0, 256)
        parts = np.split(np.arange(lay.flat_numel), world)
        got = np.concatenate([np.arange(r.start, r.stop)
                              for r in shard_flat_index(lay)])
        assert np.array_equal(got, parts[rank])


def check_invariants(lay, cap_bytes):
    A = lay.align_elems
    W = lay.world
    # tensor starts aligned, in order, non-overlapping
    end = 0
    for s, n in zip(lay.tensor_flat_off, lay.tensor_numel):
        assert s % A == 0 and s >= end
        end = s + n
    # buckets tile [0, flat) and each is a multiple of W*A, <= cap
    pos = 0
    shard = 0
    for b in lay.buckets:
        assert b.flat_off == pos and b.shard_off == shard
        assert b.numel % (W * A) == 0 and b.numel == W * b.slice_numel
        if cap_bytes > 0:
            assert b.numel * 2 <= cap_bytes
        pos += b.numel
        shard += b.slice_numel
    assert pos == lay.flat_numel and shard == lay.shard_numel
    assert lay.flat_numel >= end and lay.flat_numel - end < W * A
    # chunks: in shard order, inside their bucket slice and their tensor
    last = 0
    for c in lay.chunks:
        b = lay.buckets[c.bucket_id]
        assert b.shard_off <= c.shard_off
        assert c.shard_off + c.numel <= b.shard_off + b.slice_numel
        assert c.tensor_off + c.numel <= lay.tensor_numel[c.tensor_id]
        assert c.shard_off >= last
        last = c.shard_off + c.numel
        flat = b.flat_off + lay.rank * b.slice_numel + (c.shard_off
                                                        - b.shard_off)
        assert flat == lay.tensor_flat_off[c.tensor_id] + c.tensor_off


def test_every_tensor_element_owned_once_gpt2():
    numels = wl.gpt2_small()
    W = 8
    seen = [np.zeros(n, np.int8) for n in numels]
    for r in range(W):
        lay = build_layout(numels, W, r)
        check_invariants(lay, 25 << 20)
        for c in lay.chunks:
            seen[c.tensor_id][c.tensor_off:c.tensor_off + c.numel] += 1
    assert all((s == 1).all() for s in seen)


def test_tiny_config():
    lay = build_layout(wl.tiny(), 4, 0)
    assert sum(wl.tiny()) == 1_116_160
    assert lay.flat_numel == 1_116_160 and lay.shard_numel == 279_040
    assert len(lay.buckets) == 1
    # rank 0 owns all of tensor 0 (512x512) and the head of tensor 1
    assert as_tuples(lay) == [(0, 0, 0, 262_144, 0),
                              (1, 0, 0, 279_040 - 262_144, 262_144)]


def llama_total(L, d, kv, ffn, V):
    """Closed form of a Llama-shaped parameter count (untied, no biases)."""
    return 2 * V * d + L * (2 * d + 2 * d * d + 2 * kv * d + 3 * d * ffn) + d


def gpt2_total(L, d, ffn, V, ctx):
    return V * d + ctx * d + L * (4 * d + 4 * d * d + 3 * d + 2 * d * ffn
                                  + ffn + d + d) + 2 * d


@pytest.mark.parametrize("name,world,approx_total,approx_shard,closed", [
    ("gpt2", 8, 124e6, 15.5e6, gpt2_total(12, 768, 3072, 50257, 1024)),
    ("llama8b", 8, 8.0e9, 1.0e9, llama_total(32, 4096, 1024, 14336, 128256)),
    ("dense7b", 64, 6.7e9, 105e6, llama_total(32, 4096, 4096, 11008, 32000)),
    ("llama70b", 16, 70.6e9, 4.4e9,
     llama_total(80, 8192, 1024, 28672, 128256)),
])
def test_workload_shapes(name, world, approx_total, approx_shard, closed):
    w = wl.presets()[name]
    assert w.world == world
    total = sum(w.numels)
    assert total == closed
    assert abs(total / approx_total - 1) < 0.01
    lay = build_layout(w.numels, world, 0)
    check_invariants(lay, 25 << 20)
    assert abs(lay.shard_numel / approx_shard - 1) < 0.01
    # a full bucket is 25 MiB of bf16 whenever 25 MiB is a multiple of W*128
    assert lay.bucket_elems == 13_107_200
    assert len(lay.buckets) == -(-lay.flat_numel // 13_107_200)


def test_rejects_bad_arguments():
    with pytest.raises(LayoutError):
        build_layout([10], 0, 0)
    with pytest.raises(LayoutError):
        build_layout([10], 2, 2)
    with pytest.raises(LayoutError):
        build_layout([10], 2, 0, 25 << 20, 8)
    with pytest.raises(LayoutError):
        build_layout([-1], 2, 0)
    with pytest.raises(LayoutError):
        build_layout([10], 64, 0, 1024, 256)      # cap below W*align


def test_empty_list():
    lay = build_layout([], 4, 1)
    assert lay.flat_numel == 0 and lay.shard_numel == 0
    assert lay.buckets == [] and lay.chunks == []
    lay = build_layout([0, 0], 4, 1)
    assert lay.flat_numel == 0 and lay.chunks == []
