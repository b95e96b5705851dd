"""zs_pack_noalloc (the pack with the library's static staging, for callers
that cannot allocate) against zs_pack, the entry point it varies, through
the C-ABI: the flat all-gather buffer and every per-tensor destination,
bit for bit, on two calls in a row on one stream with no sync between them,
the second on a smaller layout (fewer chunks and tensors) so it overwrites
only part of the staging the first one left; then a third call with the
flat output alone.  Both results are also checked against the oracle's
pack.  Copies of bit patterns: the bar is bit-exact."""

import numpy as np
import pytest
import torch

import synth
import zero_sharded_optimizer_shard_amd as zs
from oracle.layout import build_layout, build_tensor_layout
from oracle.pack import pack_flat, pack_tensors
from synth import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class PackCase:
    """One rank's shard, a sentinel flat buffer and per-tensor storage (some
    tensors at odd element offsets, so both copy paths of the kernel run),
    twice: one set of destinations for zs_pack, one for zs_pack_noalloc."""

    def __init__(self, numels, W, rank, tensors, seed):
        if tensors:
            self.lay_o = build_tensor_layout(numels, W, rank)
            self.lay = zs.zs_layout_build_tensors(numels, W, rank)
        else:
            self.lay_o = build_layout(numels, W, rank)
            self.lay = zs.zs_layout_build(numels, W, rank)
        self.numels = numels
        n, F = self.lay_o.shard_numel, self.lay_o.flat_numel
        self.host_shard = synth.cpu_bits16(n, seed, synth.TAG_SENTINEL, 1,
                                           rank, 0)
        self.shard = torch.from_numpy(self.host_shard.view(np.int16)).cuda()
        self.flat0 = synth.cpu_bits16(F, seed, synth.TAG_SENTINEL, 2, 0, 0)
        self.dest = [self.destinations() for _ in range(2)]

    def destinations(self):
        flat = torch.from_numpy(self.flat0.view(np.int16)).cuda()
        bases, views = [], []
        for k, numel in enumerate(self.numels):
            off = 1 if k % 3 == 1 else 0
            base = torch.full((numel + off,), k, dtype=torch.int16,
                              device="cuda")
            bases.append(base)
            views.append(base[off:])
        return flat, views, bases

    def outputs(self, which):
        flat, views, _ = self.dest[which]
        return np16(flat), [np16(v) for v in views]

    def oracle(self):
        flat = self.flat0.copy()
        pack_flat(self.lay_o, self.host_shard, flat)
        ts = [np.full(k, t, np.uint16) for t, k in enumerate(self.numels)]
        pack_tensors(self.lay_o, self.host_shard, ts)
        return flat, ts


def run_pack(c, stream):
    flat, views, _ = c.dest[0]
    chunks = zs.zs_layout_chunks(c.lay)
    raw = np.frombuffer(zs.chunks_bytes(chunks), np.uint8).copy()
    dchunks = torch.from_numpy(raw).cuda()
    ptrs = torch.tensor([v.data_ptr() for v in views], dtype=torch.int64,
                        device="cuda")
    torch.cuda.synchronize()
    zs.zs_pack(c.lay, c.shard, flat, dchunks, len(chunks), ptrs,
               stream=stream)
    torch.cuda.synchronize()


def assert_same(a, b, what):
    fa, ta = a
    fb, tb = b
    assert np.array_equal(fa, fb), f"{what}: flat buffer"
    for k, (x, y) in enumerate(zip(ta, tb)):
        assert np.array_equal(x, y), f"{what}: tensor {k}"


def test_noalloc_pack_equals_pack_two_calls_in_a_row():
    w = wl.presets()["gpt2"]
    big = PackCase(w.numels, 8, 5, tensors=False, seed=3)
    small = PackCase([1000, 70000, 7, 129, 20000], 3, 1, tensors=True,
                     seed=4)
    assert len(small.lay_o.chunks) < len(big.lay_o.chunks)
    assert len(small.numels) < len(big.numels)
    print(f"case noalloc pack: gpt2 W=8 rank 5 ({len(big.lay_o.chunks)} "
          f"chunks), then whole-tensor W=3 rank 1 "
          f"({len(small.lay_o.chunks)} chunks)", flush=True)
    s = torch.cuda.Stream()
    for c in (big, small):
        run_pack(c, s)
    torch.cuda.synchronize()
    # the two calls in a row, one stream, no sync between them
    for c in (big, small):
        flat, views, _ = c.dest[1]
        zs.zs_pack_noalloc(c.lay, c.shard, flat, views, stream=s)
    torch.cuda.synchronize()
    for c, name in ((big, "gpt2"), (small, "whole-tensor")):
        ref = c.outputs(0)
        assert_same(c.outputs(1), ref, f"{name}: noalloc vs zs_pack")
        assert_same(ref, c.oracle(), f"{name}: zs_pack vs oracle")
    # the flat output alone, after the staging holds the small case
    out = torch.from_numpy(big.flat0.view(np.int16)).cuda()
    zs.zs_pack_noalloc(big.lay, big.shard, out, None, stream=s)
    torch.cuda.synchronize()
    assert np.array_equal(np16(out), big.outputs(0)[0])
