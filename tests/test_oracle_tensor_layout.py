"""Pins of the whole-tensor layout oracle (oracle.layout.build_tensor_layout)
against rules it does not share code with: the partition of the flat buffer,
Graham's bound for the longest-first greedy assignment against a brute-force
optimum, closed forms (equal tensors, W = 1 equals the flat mode's single
bucket), and the gather round trip of a known flat buffer."""

import itertools
import random

import numpy as np
import pytest

from oracle.layout import build_layout, build_tensor_layout
from oracle.pack import gather_tensors, pack_flat
from synth import workloads as wl


def pad(n, a=128):
    return -(-n // a) * a


@pytest.mark.parametrize("seed", range(10))
def test_partition_and_offsets(seed):
    rng = random.Random(seed)
    numels = [rng.choice([0, 1, 7, 129, 1000, 4096, 70000])
              for _ in range(rng.randint(1, 14))]
    W = rng.choice([1, 2, 3, 5, 8])
    lays = [build_tensor_layout(numels, W, r) for r in range(W)]
    F = lays[0].flat_numel
    cover = np.zeros(F, np.int32)
    seen = [0] * len(numels)
    for lay in lays:
        assert lay.owner == lays[0].owner
        off = 0
        for b, c in zip(lay.buckets, lay.chunks):
            t = c.tensor_id
            seen[t] += 1
            assert lay.owner[t] == lay.rank
            assert b.flat_off == lay.tensor_flat_off[t]
            assert b.numel == b.slice_numel == pad(numels[t])
            assert b.shard_off == off == lay.owner_shard_off[t]
            assert (c.bucket_id, c.tensor_off, c.numel, c.shard_off) == \
                (lay.buckets.index(b), 0, numels[t], off)
            cover[b.flat_off:b.flat_off + b.numel] += 1
            off += b.numel
        assert off == lay.shard_numel
    for t, n in enumerate(numels):
        assert seen[t] == (1 if n else 0)
    # the padded extents of the non-empty tensors tile the flat buffer
    assert np.all(cover == 1)


def lpt_makespan(sizes, W):
    load = [0] * W
    for t in sorted(range(len(sizes)), key=lambda t: (-sizes[t], t)):
        r = min(range(W), key=lambda q: (load[q], q))
        load[r] += sizes[t]
    return max(load)


@pytest.mark.parametrize("seed", range(12))
def test_greedy_is_within_grahams_bound_of_the_optimum(seed):
    rng = random.Random(seed)
    n = rng.randint(2, 7)
    W = rng.choice([2, 3])
    numels = [rng.randint(1, 40) * 128 for _ in range(n)]
    lays = [build_tensor_layout(numels, W, r) for r in range(W)]
    loads = [lay.shard_numel for lay in lays]
    assert max(loads) == lpt_makespan(numels, W)
    opt = min(max(sum(numels[t] for t in range(n) if a[t] == r)
                  for r in range(W))
              for a in itertools.product(range(W), repeat=n))
    assert max(loads) * 3 * W <= (4 * W - 1) * opt


def test_equal_tensors_go_one_per_rank_in_order():
    W = 8
    numels = [4096] * W
    for r in range(W):
        lay = build_tensor_layout(numels, W, r)
        assert [c.tensor_id for c in lay.chunks] == [r]
        assert lay.owner == list(range(W))


@pytest.mark.parametrize("numels,owners", [
    # all pad to 128: list order, loads tie to the lowest rank
    # (ordering by raw size would give 1, 0, 1)
    ([1, 128, 100], [0, 1, 0]),
    # all pad to 256 (raw order 250, 200, 129 would give 1, 0, 1)
    ([129, 200, 250], [0, 1, 0]),
    # pads 256, 256, 128, 128: loads 256 | 256, then 384 | 256, so the last
    # tensor goes to rank 1 (raw loads 129 | 200 would send it to rank 0)
    ([129, 200, 1, 1], [0, 1, 0, 1]),
])
def test_padding_decides_the_assignment(numels, owners):
    """Worked by hand from the rule, W = 2: sizes and loads are the sizes
    padded to the 128-element unit."""
    lays = [build_tensor_layout(numels, 2, r) for r in range(2)]
    assert lays[0].owner == owners
    for r in range(2):
        assert [c.tensor_id for c in lays[r].chunks] == \
            [t for t in range(len(numels)) if owners[t] == r]
        assert lays[r].shard_numel == sum(pad(n) for t, n in
                                          enumerate(numels) if owners[t] == r)


def test_one_rank_is_the_flat_single_bucket():
    numels = wl.tiny() + [7, 129, 70000]
    t = build_tensor_layout(numels, 1, 0)
    f = build_layout(numels, 1, 0, 0)
    assert t.shard_numel == f.shard_numel == t.flat_numel == f.flat_numel
    shard = np.arange(t.shard_numel, dtype=np.int64)
    a = np.full(t.flat_numel, -1, np.int64)
    b = np.full(f.flat_numel, -1, np.int64)
    pack_flat(t, shard, a)
    pack_flat(f, shard, b)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("W", [2, 3, 8])
def test_gather_round_trip(W):
    numels = wl.tiny() + [70000, 129, 3]
    lays = [build_tensor_layout(numels, W, r) for r in range(W)]
    F = lays[0].flat_numel
    flat = np.arange(F, dtype=np.int64) * 5 + 1
    # each rank's shard cut from the flat buffer by tensor ownership
    shards = []
    for lay in lays:
        sh = np.zeros(lay.shard_numel, np.int64)
        for b in lay.buckets:
            sh[b.shard_off:b.shard_off + b.numel] = \
                flat[b.flat_off:b.flat_off + b.numel]
        shards.append(sh)
    assert np.array_equal(gather_tensors(numels, W, shards, 0, F), flat)
    assert np.array_equal(gather_tensors(numels, W, shards, 4096, 300000),
                          flat[4096:300000])


def test_llama8b_balance():
    w = wl.presets()["llama8b"]
    loads = [build_tensor_layout(w.numels, 8, r).shard_numel
             for r in range(8)]
    total = sum(pad(n) for n in w.numels)
    assert sum(loads) == total
    # within Graham's bound of the trivial lower bound max(total/W, largest)
    lb = max(total / 8, max(w.numels))
    assert max(loads) <= (4 * 8 - 1) / (3 * 8) * lb
