"""Pins of the gather oracle (oracle.pack.gather, the ZeRO-3 / FSDP
materialisation of a flat range from every rank's shard) against rules it
does not share code with: the round trip of a known flat buffer cut into
shards by per-element ownership, and per-tensor assembly through every
rank's chunk table."""

import random

import numpy as np
import pytest

from oracle.layout import build_layout
from oracle.pack import gather, owner_runs, pack_tensors
from synth import workloads as wl


def shards_of(flat, numels, W, cap, align=256):
    """Cut a flat buffer into the W shards element by element: rank r's
    shard is its slice of every bucket, in bucket order (ownership walked
    position by position, not through pack_flat)."""
    lay0 = build_layout(numels, W, 0, cap, align)
    shards = [[] for _ in range(W)]
    pos = 0
    for b in lay0.buckets:
        for k in range(b.numel):
            shards[k // b.slice_numel].append(flat[pos + k])
        pos += b.numel
    return [np.array(s, flat.dtype) for s in shards]


@pytest.mark.parametrize("seed", range(8))
def test_round_trip_of_a_known_flat_buffer(seed):
    rng = random.Random(seed)
    numels = [rng.choice([1, 7, 129, 1000, 5000]) for _ in range(6)]
    W = rng.choice([1, 2, 3, 5, 8])
    cap = rng.choice([0, W * 256 * 3, W * 256 * 11])
    lay = build_layout(numels, W, 0, cap)
    flat = np.arange(lay.flat_numel, dtype=np.int64) * 7 + 3
    shards = shards_of(flat, numels, W, cap)
    assert np.array_equal(gather(numels, W, shards, 0, lay.flat_numel, cap),
                          flat)
    for _ in range(5):
        lo = rng.randrange(lay.flat_numel)
        hi = rng.randrange(lo, lay.flat_numel + 1)
        assert np.array_equal(gather(numels, W, shards, lo, hi, cap),
                              flat[lo:hi])
    assert gather(numels, W, shards, 3, 3, cap).size == 0


@pytest.mark.parametrize("W", [1, 3, 8])
def test_each_tensor_equals_its_chunks_from_every_rank(W):
    numels = wl.tiny() + [70000, 129]
    cap = W * 256 * 50
    lay0 = build_layout(numels, W, 0, cap)
    rng = np.random.default_rng(W)
    shards = [rng.integers(0, 1 << 16, lay0.shard_numel, dtype=np.uint16)
              for _ in range(W)]
    tensors = [np.zeros(n, np.uint16) for n in numels]
    for r in range(W):
        pack_tensors(build_layout(numels, W, r, cap), shards[r], tensors)
    for t_id, (off, n) in enumerate(zip(lay0.tensor_flat_off, numels)):
        assert np.array_equal(gather(numels, W, shards, off, off + n, cap),
                              tensors[t_id])


@pytest.mark.parametrize("seed", range(6))
def test_owner_runs_agree_with_gather(seed):
    rng = random.Random(100 + seed)
    numels = [rng.choice([7, 129, 1000, 5000]) for _ in range(5)]
    W = rng.choice([1, 2, 5, 8])
    cap = rng.choice([0, W * 256 * 4])
    lay = build_layout(numels, W, rng.randrange(W), cap)
    shards = [np.random.default_rng(r).integers(0, 1 << 16, lay.shard_numel,
                                                dtype=np.uint16)
              for r in range(W)]
    lo = rng.randrange(lay.flat_numel)
    hi = rng.randrange(lo, lay.flat_numel + 1)
    want = gather(numels, W, shards, lo, hi, cap)
    got = np.empty(hi - lo, np.uint16)
    covered = 0
    for a, n, r, s0 in owner_runs(lay, lo, hi):
        got[a - lo:a - lo + n] = shards[r][s0:s0 + n]
        covered += n
    assert covered == hi - lo
    assert np.array_equal(got, want)
