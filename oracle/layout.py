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
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence


def _roundup(x: int, a: int) -> int:
    return ((x + a - 1) // a) * a


@dataclass
class Bucket:
    flat_off: int
    numel: int
    slice_numel: int
    shard_off: int


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
                 align_bytes: int = 256) -> Layout:
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
    while off < content_end:
        numel = min(full, _roundup(content_end - off, unit))
        sl = numel // world
        buckets.append(Bucket(off, numel, sl, shard_off))
        off += numel
        shard_off += sl
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
                  buckets=buckets, chunks=chunks)


def shard_flat_index(lay: Layout) -> List[range]:
    """The flat positions of the rank's shard, one range per bucket slice."""
    return [range(b.flat_off + lay.rank * b.slice_numel,
                  b.flat_off + (lay.rank + 1) * b.slice_numel)
            for b in lay.buckets]


def build_tensor_layout(tensor_numel: Sequence[int], world: int, rank: int,
                        align_bytes: int = 256) -> Layout:
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
    for t in range(len(tensor_numel)):
        if owner[t] != rank or tensor_numel[t] == 0:
            continue
        b_id = len(buckets)
        buckets.append(Bucket(starts[t], padded[t], padded[t], owner_off[t]))
        chunks.append(Chunk(t, b_id, 0, tensor_numel[t], owner_off[t]))
    return Layout(world=world, rank=rank, align_elems=align, bucket_elems=0,
                  tensor_numel=list(tensor_numel), tensor_flat_off=starts,
                  flat_numel=flat_numel, shard_numel=fill[rank],
                  buckets=buckets, chunks=chunks,
                  whole_tensors=True, owner=owner,
                  owner_shard_off=owner_off)
