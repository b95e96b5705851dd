"""Pins of the tests' statement of the library's tiled storage format
(tests/tiles.py): the tile of every shard element against a walk of the
shard that opens tiles one element at a time, the per-bucket tile offsets,
and round trips of the tiled state and gradients."""

import random

import numpy as np
import pytest

from oracle.layout import build_layout
from synth import workloads as wl
from tiles import (TILE, from_tiled_state, n_tiles, tile_offsets, tile_slot,
                   to_tiled_grads, to_tiled_state)


def tiles_by_filling(lay, T):
    """Tile of every shard element by the operational rule: walk the shard
    in order, start a new tile at every bucket boundary and whenever the
    current tile holds T elements."""
    out = []
    tile, fill = -1, T
    for b in lay.buckets:
        fill = T                        # a bucket never shares a tile
        for _ in range(b.slice_numel):
            if fill == T:
                tile += 1
                fill = 0
            out.append(tile * T + fill)
            fill += 1
    return np.array(out, np.int64), tile + 1


@pytest.mark.parametrize("seed", range(12))
def test_tile_slots_by_filling(seed):
    rng = random.Random(seed)
    numels = [rng.choice([7, 129, 1000, 20000, 70000]) for _ in range(6)]
    W = rng.choice([1, 2, 3, 8])
    cap = rng.choice([0, W * 256 * 37, W * 256 * 100])
    lay = build_layout(numels, W, rng.randrange(W), cap)
    for T in (TILE, 256):               # the rule at the real and a small T
        want, count = tiles_by_filling(lay, T)
        assert n_tiles(lay, T) == count
        assert np.array_equal(tile_slot(lay, T), want)
        # each bucket's first tile is where the walk opened it
        for b, t0 in zip(lay.buckets, tile_offsets(lay, T)):
            if b.slice_numel:
                assert want[b.shard_off] == t0 * T


def test_tile_layout_invariants_workloads():
    for name in ("tiny", "gpt2", "llama8b", "dense7b", "llama70b"):
        w = wl.presets()[name]
        lay = build_layout(w.numels, w.world, 0)
        offs = tile_offsets(lay)
        tiles = 0
        for b, t0 in zip(lay.buckets, offs):
            assert t0 == tiles
            tiles += -(-b.slice_numel // TILE)
        assert tiles == n_tiles(lay)
        # tiled buffers waste less than one tile per bucket
        assert n_tiles(lay) * TILE - lay.shard_numel < TILE * len(lay.buckets)


def test_tiled_state_and_grads_round_trip():
    lay = build_layout([1000, 70000, 129, 20000], 3, 1, 3 * 256 * 50)
    n = lay.shard_numel
    nt = n_tiles(lay)
    rng = np.random.default_rng(0)
    ma, m, v = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
    st = to_tiled_state(lay, ma, m, v)
    assert st.size == nt * 3 * TILE
    back = from_tiled_state(lay, st)
    for x, y in zip(back, (ma, m, v)):
        assert np.array_equal(x, y)
    # every non-slot position is padding (zero), and each slot holds its
    # element's value in the master row
    slot = tile_slot(lay)
    mask = np.zeros(nt * TILE, bool)
    mask[slot] = True
    assert np.count_nonzero(mask) == n
    st3 = st.reshape(nt, 3, TILE)
    assert not st3[:, 0, :].reshape(-1)[~mask].any()
    assert np.array_equal(st3[:, 0, :].reshape(-1)[slot], ma)
    G = rng.integers(0, 1 << 16, (3, n), dtype=np.uint16)
    tg = to_tiled_grads(lay, G).reshape(nt, 3, TILE)
    for s in range(3):
        assert np.array_equal(tg[:, s, :].reshape(-1)[slot], G[s])
        assert not tg[:, s, :].reshape(-1)[~mask].any()
