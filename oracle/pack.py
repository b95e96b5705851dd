"""Pack and gather oracles: the local half of the all-gather, and the
ZeRO-3 / FSDP materialisation of a layer from every rank's shard.

TEST INFRASTRUCTURE: see oracle/__init__.py.

The all-gather of the CS336 lecture 8 notes ("ZeRO-1 code example", last
step) concatenates every rank's updated slice in rank order.  One rank's part
of that result is its own slices placed at their flat positions: bucket b's
slice of rank r goes to [b.flat_off + r*b.slice_numel, +b.slice_numel).  The
per-tensor form writes the same values into each tensor's own storage through
the chunk table (tensor view = flat buffer at the tensor's start).
"""

from __future__ import annotations

import numpy as np

from .layout import Layout, build_layout, build_tensor_layout


def pack_flat(lay: Layout, shard: np.ndarray, full_flat: np.ndarray) -> None:
    """Write the rank's shard into its positions of the flat buffer (in the
    whole-tensor mode, each owned tensor at its flat offset)."""
    for b in lay.buckets:
        dst = b.flat_off + (0 if lay.whole_tensors
                            else lay.rank * b.slice_numel)
        full_flat[dst:dst + b.slice_numel] = \
            shard[b.shard_off:b.shard_off + b.slice_numel]


def pack_tensors(lay: Layout, shard: np.ndarray, tensors: list) -> None:
    """Write the rank's shard into per-tensor arrays through the chunk table."""
    for c in lay.chunks:
        tensors[c.tensor_id][c.tensor_off:c.tensor_off + c.numel] = \
            shard[c.shard_off:c.shard_off + c.numel]


def gather(tensor_numel, world: int, shards, flat_lo: int, flat_hi: int,
           bucket_cap_bytes: int = 25 << 20,
           align_bytes: int = 256) -> np.ndarray:
    """The flat range [flat_lo, flat_hi) of the bf16 parameters, assembled
    from the shards of all `world` ranks (shards[r]: rank r's bf16 shard).

    ZeRO-3 / FSDP keep only a shard of every weight per rank and all-gather
    a layer's full weight just before it is used (podcast summary of "Training
    at thousands of GPUs", section "ZeRO optimizer"; CS336 lecture 8 notes,
    "Code example: FSDP").  The all-gather concatenates the ranks' slices in
    rank order, so the full flat buffer is every rank's shard written back at
    its flat positions; the layer is a window of it."""
    lays = [build_layout(tensor_numel, world, r, bucket_cap_bytes,
                         align_bytes) for r in range(world)]
    return _gather(lays, shards, flat_lo, flat_hi)


def gather_tensors(tensor_numel, world: int, shards, flat_lo: int,
                   flat_hi: int, align_bytes: int = 256) -> np.ndarray:
    """The gather of the whole-tensor mode: every tensor comes whole from
    its owner's shard (a broadcast from the owner instead of an all-gather
    of slices)."""
    lays = [build_tensor_layout(tensor_numel, world, r, align_bytes)
            for r in range(world)]
    return _gather(lays, shards, flat_lo, flat_hi)


def _gather(lays, shards, flat_lo, flat_hi):
    full = np.zeros(lays[0].flat_numel, np.asarray(shards[0]).dtype)
    for lay, sh in zip(lays, shards):
        pack_flat(lay, np.asarray(sh), full)
    return full[flat_lo:flat_hi].copy()


def owner_runs(lay: Layout, flat_lo: int, flat_hi: int):
    """The flat range [flat_lo, flat_hi) as runs (flat_start, numel, rank,
    shard_start): each run lies in one rank's slice of one bucket, and its
    values are that rank's shard from shard_start on.  `lay` may be any
    rank's layout (the bucket table is the same for all)."""
    runs = []
    for b in lay.buckets:
        for r in range(lay.world):
            s0 = b.flat_off + r * b.slice_numel
            a, e = max(s0, flat_lo), min(s0 + b.slice_numel, flat_hi)
            if e > a:
                runs.append((a, e - a, r, b.shard_off + (a - s0)))
    return runs
