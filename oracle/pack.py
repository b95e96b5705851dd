"""Pack oracle: the local half of the all-gather.

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

from .layout import Layout


def pack_flat(lay: Layout, shard: np.ndarray, full_flat: np.ndarray) -> None:
    """Write the rank's shard into its positions of the flat buffer."""
    for b in lay.buckets:
        dst = b.flat_off + lay.rank * b.slice_numel
        full_flat[dst:dst + b.slice_numel] = \
            shard[b.shard_off:b.shard_off + b.slice_numel]


def pack_tensors(lay: Layout, shard: np.ndarray, tensors: list) -> None:
    """Write the rank's shard into per-tensor arrays through the chunk table."""
    for c in lay.chunks:
        tensors[c.tensor_id][c.tensor_off:c.tensor_off + c.numel] = \
            shard[c.shard_off:c.shard_off + c.numel]
