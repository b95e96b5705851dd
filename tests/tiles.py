"""The library's tiled storage format, stated independently for the tests.

The tiled HBM layouts of the optimizer state and of the gradient slices are
a storage choice of the HIP library, not part of the method, so they live
here beside the tests rather than in the oracle.  The rule: each bucket's
slice of the rank's shard is cut into TILE-element tiles, the last one
padded; tiles are numbered across buckets in bucket order (a bucket never
shares a tile with another).  Tiled state: tile i holds rows [master | m |
v] (or [m | v] for the pure-bf16 step) of TILE floats each.  Tiled
gradients: tile i holds source ranks 0..W-1, TILE bf16 values each.
Padding positions are zero.

Every function takes a layout object of the oracle (oracle.layout.Layout):
only its buckets' slice_numel and shard_off are read.  The mapping is
pinned by tests/test_tiles.py against a walk of the shard that opens tiles
one element at a time.
"""

from __future__ import annotations

import numpy as np

TILE = 8192          # elements per tile


def tile_offsets(lay, tile: int = TILE):
    """First tile of every bucket's slice, in bucket order."""
    out, tiles = [], 0
    for b in lay.buckets:
        out.append(tiles)
        tiles += -(-b.slice_numel // tile)
    return out


def n_tiles(lay, tile: int = TILE) -> int:
    return sum(-(-b.slice_numel // tile) for b in lay.buckets)


def tile_slot_range(lay, bucket_id: int, j0: int, k: int, tile: int = TILE):
    """int64 [k]: tile * T + position, in the tiled layouts (T = tile), of
    elements j0 .. j0+k-1 of bucket bucket_id's slice: element j sits in
    the bucket's first tile + j // T at position j % T."""
    b = lay.buckets[bucket_id]
    if j0 < 0 or j0 + k > b.slice_numel:
        raise IndexError("range outside the bucket's slice")
    t0 = tile_offsets(lay, tile)[bucket_id]
    j = np.arange(j0, j0 + k, dtype=np.int64)
    return (t0 + j // tile) * tile + j % tile


def tile_slot(lay, tile: int = TILE) -> np.ndarray:
    """int64 [shard_numel]: tile * T + position of every shard element in
    the tiled layouts."""
    out = np.empty(lay.shard_numel, np.int64)
    offs = tile_offsets(lay, tile)
    for b, t0 in zip(lay.buckets, offs):
        j = np.arange(b.slice_numel, dtype=np.int64)
        out[b.shard_off:b.shard_off + b.slice_numel] = \
            (t0 + j // tile) * tile + j % tile
    return out


def to_tiled_rows(lay, rows) -> np.ndarray:
    """Plain fp32 arrays [shard_numel], one per row, -> a tiled state
    [n_tiles * len(rows) * TILE]; padding positions 0."""
    R = len(rows)
    nt = n_tiles(lay)
    st = np.zeros((nt, R, TILE), np.float32)
    slot = tile_slot(lay)
    t, p = slot // TILE, slot % TILE
    for k, a in enumerate(rows):
        st[t, k, p] = a
    return st.reshape(-1)


def from_tiled_rows(lay, state, n_rows: int):
    """A tiled state of n_rows rows -> the plain arrays, one per row."""
    st = np.asarray(state, np.float32).reshape(n_tiles(lay), n_rows, TILE)
    slot = tile_slot(lay)
    t, p = slot // TILE, slot % TILE
    return tuple(st[t, k, p].copy() for k in range(n_rows))


def to_tiled_state(lay, master, m, v) -> np.ndarray:
    """Plain fp32 master/m/v [shard_numel] -> tiled state; padding 0."""
    return to_tiled_rows(lay, [master, m, v])


def from_tiled_state(lay, state):
    """Tiled state -> plain (master, m, v)."""
    return from_tiled_rows(lay, state, 3)


def to_tiled_grads(lay, G) -> np.ndarray:
    """Gradient slices uint16 [W][shard_numel] -> tiled [n_tiles*W*TILE];
    padding positions 0."""
    W = lay.world
    out = np.zeros((n_tiles(lay), W, TILE), np.uint16)
    slot = tile_slot(lay)
    t, p = slot // TILE, slot % TILE
    for s in range(W):
        out[t, s, p] = G[s]
    return out.reshape(-1)
