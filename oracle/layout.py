"""Layout oracle: flat buffer, fixed-size buckets, per-rank slices and chunks.

TEST INFRASTRUCTURE. Only tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module. The product path never does.

What it computes (plain Python loops, no cleverness, shares nothing with the
HIP library):

* Every tensor of the parameter list starts on an ``align_bytes`` boundary of a
  flat bf16 buffer, in list order.  The pages flatten the parameters before
  sharding them (podcast summary of N. Tazi's "Training at thousands of GPUs",
  section "ZeRO optimizer", the FSDP1 remark) and keep the gradients in one
  contiguous buffer (DDP-to-ZeRO blog, section 3.3, the
  ``contiguous_gradients`` knob of the DeepSpeed config).
* The flat buffer is cut into buckets of ``bucket_cap_mb`` (25 MiB of bf16 by
  default; podcast summary, section "Data parallelism", and DDP-to-ZeRO blog,
  section 2.1).  Reading taken: a bucket is a fixed window of the flat buffer
  that may cut through tensors; full buckets hold the largest multiple of
  ``world * align_elems`` elements that fits under the cap; the last bucket
  holds the remainder rounded up to that unit; the rounding is zero padding.
* Each bucket is reduce-scattered ``world`` ways and rank r owns the r-th
  contiguous slice of it (CS336 lecture 8 notes, "ZeRO-1 code example":
  reduce-scatter gives each rank its own chunk; all-gather concatenates the
  chunks in rank order).  A rank's shard is its slices concatenated in bucket
  order.
* The chunk table lists, for one rank, the maximal runs of its shard that lie
  inside one tensor: (tensor_id, bucket_id, tensor_off, numel, shard_off).
  Padding is in no chunk.
* Tiles.  The tiled HBM layouts of the optimizer state and of the gradient
  slices are a storage format of the implementation, not part of the method;
  they are stated here so that tests can place and read values in them
  without the library.  Each bucket's slice is cut into ``TILE``-element
  tiles, the last one padded; tiles are numbered across buckets in bucket
  order (``Bucket.tile_off`` is the first tile of the slice).  Tiled state:
  tile i holds ``[master | m | v]`` of ``TILE`` floats each.  Tiled
  gradients: tile i holds source ranks 0..W-1, ``TILE`` bf16 values each.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np

TILE = 8192          # elements per tile of the tiled layouts


def _roundup(x: int, a: int) -> int:
    return ((x + a - 1) // a) * a


@dataclass
class Bucket:
    flat_off: int
    numel: int
    slice_numel: int
    shard_off: int
    tile_off: int = 0


@dataclass
class Chunk:
    tensor_id: int
    bucket_id: int
    tensor_off: int
    numel: int
    shard_off: int


@dataclass
class Layout:
    world: int
    rank: int
    align_elems: int
    bucket_elems: int          # size of a full bucket, in elements
    tensor_numel: List[int]
    tensor_flat_off: List[int]
    flat_numel: int
    shard_numel: int
    n_tiles: int = 0
    tile: int = TILE
    buckets: List[Bucket] = field(default_factory=list)
    chunks: List[Chunk] = field(default_factory=list)
    # whole-tensor mode: the owner rank of every tensor and its offset in
    # the owner's shard (empty lists in the flat mode)
    whole_tensors: bool = False
    owner: List[int] = field(default_factory=list)
    owner_shard_off: List[int] = field(default_factory=list)


class LayoutError(ValueError):
    pass


def build_layout(tensor_numel: Sequence[int], world: int, rank: int,
                 bucket_cap_bytes: int = 25 << 20,
                 align_bytes: int = 256, tile: int = TILE) -> Layout:
    """Build the layout of one rank.  See the module docstring for the rule.

    ``bucket_cap_bytes <= 0`` means one bucket holding the whole flat buffer,
    which is the unbucketed reduce-scatter of the CS336 ZeRO-1 sketch.
    """
    if world < 1 or not (0 <= rank < world):
        raise LayoutError("need world >= 1 and 0 <= rank < world")
    if align_bytes < 16 or align_bytes % 16:
        raise LayoutError("align_bytes must be a positive multiple of 16")
    for n in tensor_numel:
        if n < 0:
            raise LayoutError("negative tensor numel")
    align = align_bytes // 2               # bf16 elements per alignment unit

    # 1. tensor starts: each one rounded up to the alignment unit
    starts = []
    pos = 0
    for n in tensor_numel:
        pos = _roundup(pos, align)
        starts.append(pos)
        pos += n
    content_end = pos

    # 2. bucket size
    unit = world * align
    if bucket_cap_bytes <= 0:
        full = max(_roundup(content_end, unit), unit)
    else:
        full = ((bucket_cap_bytes // 2) // unit) * unit
        if full == 0:
            raise LayoutError("bucket cap smaller than world * align")

    # 3. buckets: fixed windows, the last one rounded up to the unit
    buckets = []
    off = 0
    shard_off = 0
    tiles = 0
    while off < content_end:
        numel = min(full, _roundup(content_end - off, unit))
        sl = numel // world
        buckets.append(Bucket(off, numel, sl, shard_off, tiles))
        off += numel
        shard_off += sl
        tiles += _roundup(sl, tile) // tile
    flat_numel = off
    shard_numel = shard_off

    # 4. chunks of this rank: every (bucket, tensor) intersection, in order
    chunks = []
    for b_id, b in enumerate(buckets):
        lo = b.flat_off + rank * b.slice_numel
        hi = lo + b.slice_numel
        for t_id, (t0, n) in enumerate(zip(starts, tensor_numel)):
            s = max(lo, t0)
            e = min(hi, t0 + n)
            if e > s:
                chunks.append(Chunk(t_id, b_id, s - t0, e - s,
                                    b.shard_off + (s - lo)))

    return Layout(world=world, rank=rank, align_elems=align, bucket_elems=full,
                  tensor_numel=list(tensor_numel), tensor_flat_off=starts,
                  flat_numel=flat_numel, shard_numel=shard_numel,
                  n_tiles=tiles, tile=tile, buckets=buckets, chunks=chunks)


def shard_flat_index(lay: Layout) -> List[range]:
    """The flat positions of the rank's shard, one range per bucket slice."""
    return [range(b.flat_off + lay.rank * b.slice_numel,
                  b.flat_off + (lay.rank + 1) * b.slice_numel)
            for b in lay.buckets]


def tile_slot_range(lay: Layout, bucket_id: int, j0: int, k: int):
    """int64 [k]: tile * T + position, in the tiled layouts (T = lay.tile),
    of elements j0 .. j0+k-1 of bucket bucket_id's slice: element j sits in
    tile b.tile_off + j // T at position j % T."""
    b = lay.buckets[bucket_id]
    if j0 < 0 or j0 + k > b.slice_numel:
        raise IndexError("range outside the bucket's slice")
    T = lay.tile
    j = np.arange(j0, j0 + k, dtype=np.int64)
    return (b.tile_off + j // T) * T + j % T


def tile_slot(lay: Layout) -> np.ndarray:
    """int64 [shard_numel]: tile * T + position of every shard element in
    the tiled layouts (see tile_slot_range)."""
    out = np.empty(lay.shard_numel, np.int64)
    for b_id, b in enumerate(lay.buckets):
        out[b.shard_off:b.shard_off + b.slice_numel] = \
            tile_slot_range(lay, b_id, 0, b.slice_numel)
    return out


def to_tiled_rows(lay: Layout, rows) -> np.ndarray:
    """Plain fp32 arrays [shard_numel], one per row, -> a tiled state
    [n_tiles * len(rows) * lay.tile]; padding positions 0."""
    R = len(rows)
    st = np.zeros((lay.n_tiles, R, lay.tile), np.float32)
    slot = tile_slot(lay)
    t, p = slot // lay.tile, slot % lay.tile
    for k, a in enumerate(rows):
        st[t, k, p] = a
    return st.reshape(-1)


def from_tiled_rows(lay: Layout, state, n_rows: int):
    """A tiled state of n_rows rows -> the plain arrays, one per row."""
    st = np.asarray(state, np.float32).reshape(lay.n_tiles, n_rows, lay.tile)
    slot = tile_slot(lay)
    t, p = slot // lay.tile, slot % lay.tile
    return tuple(st[t, k, p].copy() for k in range(n_rows))


def to_tiled_state(lay: Layout, master, m, v) -> np.ndarray:
    """Plain fp32 master/m/v [shard_numel] -> tiled state
    [n_tiles * 3 * lay.tile]; padding positions 0."""
    return to_tiled_rows(lay, [master, m, v])


def from_tiled_state(lay: Layout, state):
    """Tiled state -> plain (master, m, v)."""
    return from_tiled_rows(lay, state, 3)


def to_tiled_grads(lay: Layout, G) -> np.ndarray:
    """Gradient slices uint16 [W][shard_numel] -> tiled [n_tiles*W*lay.tile];
    padding positions 0."""
    W = lay.world
    out = np.zeros((lay.n_tiles, W, lay.tile), np.uint16)
    slot = tile_slot(lay)
    t, p = slot // lay.tile, slot % lay.tile
    for s in range(W):
        out[t, s, p] = G[s]
    return out.reshape(-1)


def build_tensor_layout(tensor_numel: Sequence[int], world: int, rank: int,
                        align_bytes: int = 256,
                        tile: int = TILE) -> Layout:
    """Whole-tensor shard assignment (podcast summary of "Training at
    thousands of GPUs", section "ZeRO optimizer": an optimizer that needs
    whole tensors, such as Muon, cannot work on flattened slices; the
    shards are assigned at whole-tensor granularity, as FSDP2 keeps whole
    tensors per rank).

    Reading: every tensor belongs entirely to one rank.  Tensors are
    assigned greedily, longest first: in order of decreasing padded size
    (ties by list index), each goes to the rank with the least padded load
    so far (ties to the lowest rank).  A rank's shard is its tensors in list
    order, each padded to the alignment unit; one bucket per owned non-empty
    tensor, whose whole extent is this rank's slice, at the tensor's flat
    offset.  The flat buffer is the same aligned flattening as the flat
    mode, rounded up to the alignment unit; the padded tensors partition
    it."""
    if world < 1 or not (0 <= rank < world):
        raise LayoutError("need world >= 1 and 0 <= rank < world")
    if align_bytes < 16 or align_bytes % 16:
        raise LayoutError("align_bytes must be a positive multiple of 16")
    for n in tensor_numel:
        if n < 0:
            raise LayoutError("negative tensor numel")
    align = align_bytes // 2
    starts = []
    pos = 0
    for n in tensor_numel:
        pos = _roundup(pos, align)
        starts.append(pos)
        pos += n
    flat_numel = _roundup(pos, align)
    padded = [_roundup(n, align) for n in tensor_numel]

    # greedy assignment, longest first
    order = sorted(range(len(tensor_numel)), key=lambda t: (-padded[t], t))
    load = [0] * world
    owner = [0] * len(tensor_numel)
    for t in order:
        r = min(range(world), key=lambda q: (load[q], q))
        owner[t] = r
        load[r] += padded[t]
    # shard offsets inside each owner's shard, in list order
    fill = [0] * world
    owner_off = [0] * len(tensor_numel)
    for t in range(len(tensor_numel)):
        owner_off[t] = fill[owner[t]]
        fill[owner[t]] += padded[t]

    buckets, chunks = [], []
    tiles = 0
    for t in range(len(tensor_numel)):
        if owner[t] != rank or tensor_numel[t] == 0:
            continue
        b_id = len(buckets)
        buckets.append(Bucket(starts[t], padded[t], padded[t], owner_off[t],
                              tiles))
        chunks.append(Chunk(t, b_id, 0, tensor_numel[t], owner_off[t]))
        tiles += _roundup(padded[t], tile) // tile
    return Layout(world=world, rank=rank, align_elems=align, bucket_elems=0,
                  tensor_numel=list(tensor_numel), tensor_flat_off=starts,
                  flat_numel=flat_numel, shard_numel=fill[rank],
                  n_tiles=tiles, tile=tile, buckets=buckets, chunks=chunks,
                  whole_tensors=True, owner=owner,
                  owner_shard_off=owner_off)
