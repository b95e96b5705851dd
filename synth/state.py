"""Seeded synthetic optimizer inputs for one rank, on the host (numpy) or on
the device (torch tensors as plain memory), from the shared generator.

Keys: gradients of source rank s at step t use (seed, TAG_GRAD, t, s) and the
shard index; the fp32 master uses (seed, TAG_MASTER, 0, 0) and the shard
index; m and v start at zero unless warm values are asked for.  Padding
positions of the shard (in no chunk of the layout) are zero in every array.
Nothing here computes any part of the optimizer step.
"""

from __future__ import annotations

import numpy as np

from . import (TAG_GRAD, TAG_M, TAG_MASTER, TAG_V, cpu_normal_bf16,
               cpu_normal_f32, dev_normal_bf16, dev_normal_f32)


def padding_runs(shard_numel, chunks):
    """Shard ranges covered by no chunk, as (start, stop) pairs.  `chunks`
    are objects with shard_off and numel, sorted by shard_off."""
    runs = []
    pos = 0
    for c in chunks:
        if c.shard_off > pos:
            runs.append((pos, c.shard_off))
        pos = max(pos, c.shard_off + c.numel)
    if pos < shard_numel:
        runs.append((pos, shard_numel))
    return runs


def _clip_runs(runs, a, n):
    out = []
    for s, e in runs:
        s2, e2 = max(s, a), min(e, a + n)
        if e2 > s2:
            out.append((s2 - a, e2 - a))
    return out


# ---- host ---------------------------------------------------------------------

def cpu_grads(W, a, n, step, sigma, seed=0, pad=()):
    """uint16 [W][n]: bf16 gradients of shard elements [a, a+n)."""
    G = np.stack([cpu_normal_bf16(n, seed, TAG_GRAD, step, s, a, sigma)
                  for s in range(W)]) if W else np.zeros((0, n), np.uint16)
    for s0, e0 in _clip_runs(pad, a, n):
        G[:, s0:e0] = 0
    return G


def cpu_state(a, n, master_sigma, seed=0, pad=(), warm=None):
    """fp32 master, m, v of shard elements [a, a+n).  warm=(m_sigma,
    v_sigma) draws nonzero moments (v as |N|) instead of zeros."""
    master = cpu_normal_f32(n, seed, TAG_MASTER, 0, 0, a, master_sigma)
    if warm:
        m = cpu_normal_f32(n, seed, TAG_M, 0, 0, a, warm[0])
        v = cpu_normal_f32(n, seed, TAG_V, 0, 0, a, warm[1], absval=True)
    else:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    for s0, e0 in _clip_runs(pad, a, n):
        master[s0:e0] = 0
        m[s0:e0] = 0
        v[s0:e0] = 0
    return master, m, v


# ---- device -------------------------------------------------------------------

def dev_grads(out, W, n, step, sigma, seed=0, pad=(), stream=None):
    """Fill out[:W, :n] (a [W][stride] 2-byte tensor) with the gradients of
    shard elements [0, n)."""
    for s in range(W):
        dev_normal_bf16(out[s, :n], seed, TAG_GRAD, step, s, 0, sigma,
                        stream=stream)
        for s0, e0 in pad:
            out[s, s0:e0].zero_()


def dev_state(master, m, v, master_sigma, seed=0, pad=(), warm=None,
              stream=None):
    dev_normal_f32(master, seed, TAG_MASTER, 0, 0, 0, master_sigma,
                   stream=stream)
    if warm:
        dev_normal_f32(m, seed, TAG_M, 0, 0, 0, warm[0], stream=stream)
        dev_normal_f32(v, seed, TAG_V, 0, 0, 0, warm[1], absval=True,
                       stream=stream)
    else:
        m.zero_()
        v.zero_()
    for s0, e0 in pad:
        master[s0:e0].zero_()
        m[s0:e0].zero_()
        v[s0:e0].zero_()
