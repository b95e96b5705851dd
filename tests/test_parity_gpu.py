"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Every case runs the same seeded inputs through both sides and compares
every element (small and GPT-2-sized shards) or sampled windows (the
Llama-3-8B-shaped and 7B-shaped shards at full size, in the launch
configuration the benchmark times).  The step is elementwise, so a window
is checked independently of the rest of the shard.

The GPU keeps the optimizer state in the tiled layout; results are read
back through an independent statement of the tile mapping, so the
placement is checked as well as the arithmetic.  The tile mapping is the
tests' own statement of the library's storage format (tests/tiles.py).
"""

import random

import numpy as np
import pytest
import torch

import synth
import zero_sharded_optimizer_shard_amd as zs
from oracle import step as O
from oracle.layout import build_layout, build_tensor_layout
from oracle.pack import (gather, gather_tensors, owner_runs, pack_flat,
                         pack_tensors)
from synth import state as S
from synth import workloads as wl

from parity import assert_parity
from tiles import (TILE, from_tiled_rows, from_tiled_state, n_tiles,
                   tile_offsets, tile_slot, tile_slot_range, to_tiled_grads,
                   to_tiled_rows, to_tiled_state)

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
OHP = O.AdamW(**HP)
LAYOUTS = ["slices", "tiled"]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(*a):
    print(*a, flush=True)


def dev_bf16(n):
    return torch.empty(n, dtype=torch.bfloat16, device="cuda")


def dev_f32(n):
    return torch.empty(n, dtype=torch.float32, device="cuda")


def np16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def npf(t):
    return t.cpu().numpy()


def dev_state(lay, lay_o, sigma, seed=0, pad=(), warm=None):
    """Tiled state on the device from the seeded plain arrays."""
    n = lay_o.shard_numel
    master, m, v = dev_f32(n), dev_f32(n), dev_f32(n)
    S.dev_state(master, m, v, sigma, seed, pad, warm)
    state = dev_f32(n_tiles(lay_o) * 3 * TILE)
    state.fill_(float("nan"))             # padding must be overwritten
    zs.zs_state_pack(lay, master, m, v, state)
    return state


def read_state(lay_o, state):
    return from_tiled_state(lay_o, npf(state))


def dev_tiled_bucket(full, lay_o, b_id):
    """Bucket b_id's gradients in the tiled staging form ([tiles][W][TILE]
    bf16, padding zero), cut from the plain device slices full [W][>= n]
    by tensor indexing alone (the rule of tests/tiles.py)."""
    b = lay_o.buckets[b_id]
    W = full.shape[0]
    tb = -(-b.slice_numel // TILE)
    tmp = torch.zeros((W, tb * TILE), dtype=full.dtype, device=full.device)
    tmp[:, :b.slice_numel] = full[:, b.shard_off:b.shard_off + b.slice_numel]
    return tmp.view(W, tb, TILE).permute(1, 0, 2).contiguous().view(-1)


class Case:
    """One rank's step on the GPU and on the oracle, full arrays.

    gpu=False keeps only the oracle's side (the layouts and the host
    arrays): tests of other entry points run their own device side on the
    same seeded inputs (dev_state / dev_grads with this case's seed and
    padding) and compare with check()."""

    def __init__(self, numels, W, rank, cap=25 << 20, align=256, sigma=1e-3,
                 stride_pad=0, warm=None, seed=0, layout="slices",
                 tensors=False, gpu=True):
        if tensors:                         # whole-tensor shard assignment
            self.lay_o = build_tensor_layout(numels, W, rank, align)
            self.lay = zs.zs_layout_build_tensors(numels, W, rank, align)
        else:
            self.lay_o = build_layout(numels, W, rank, cap, align)
            self.lay = zs.zs_layout_build(numels, W, rank, cap, align)
        self.W, self.rank, self.sigma, self.seed = W, rank, sigma, seed
        self.layout = layout
        self.warm = warm
        n = self.n = self.lay_o.shard_numel
        self.stride = n + stride_pad
        self.pad = S.padding_runs(n, self.lay_o.chunks)
        self.om, self.omm, self.ov = S.cpu_state(0, n, 0.02, seed, self.pad,
                                                 warm)
        self.op = None
        if not gpu:
            return
        self.G = torch.empty((W, self.stride), dtype=torch.bfloat16,
                             device="cuda")
        self.G.view(torch.int16).fill_(0x7fc0)      # NaN beyond n: never read
        if layout == "tiled":
            self.Gt = dev_bf16(max(n_tiles(self.lay_o) * W * TILE, 1))
        self.state = dev_state(self.lay, self.lay_o, 0.02, seed, self.pad,
                               warm)
        self.p = dev_bf16(n)

    def dev_state(self):
        """A fresh tiled device state with this case's initial values."""
        return dev_state(self.lay, self.lay_o, 0.02, self.seed, self.pad,
                         self.warm)

    def dev_grads(self, out, t):
        """This case's step-t gradients into out[:W, :n] on the device."""
        S.dev_grads(out, self.W, self.n, t, self.sigma, self.seed, self.pad)

    def oracle_step(self, t, hp=None):
        """Advance the oracle's arrays by step t; returns its bf16 shard."""
        hp = HP if hp is None else hp
        Gc = S.cpu_grads(self.W, 0, self.n, t, self.sigma, self.seed,
                         self.pad)
        self.op = O.step(Gc, self.om, self.omm, self.ov, O.AdamW(**hp), t)
        return self.op

    def check(self, state, where, p=None, flat=None, flat_before=None):
        """The device tiled state, and the bf16 shard p and/or the flat
        buffer (flat_before: its host contents before the steps), against
        the oracle's arrays after its last step, bit for bit."""
        torch.cuda.synchronize()
        ma, m, v = read_state(self.lay_o, state)
        got = dict(master=ma, m=m, v=v)
        want = dict(master=self.om, m=self.omm, v=self.ov)
        if p is not None:
            got["p"], want["p"] = np16(p), self.op
        assert_parity(got, want, where)
        if flat is not None:
            ref = flat_before.copy()
            pack_flat(self.lay_o, self.op, ref)
            assert np.array_equal(np16(flat), ref), f"{where}: flat buffer"

    def step(self, t, full_flat=None, check=True, exact=True, hp=None):
        hp = HP if hp is None else hp
        S.dev_grads(self.G, self.W, self.n, t, self.sigma, self.seed,
                    self.pad)
        if self.layout == "tiled":
            zs.zs_grads_tile(self.lay, -1, self.G, self.stride, self.Gt)
            zs.zs_step(self.lay, self.Gt, self.state, self.p, full_flat,
                       grad_layout="tiled", step=t, **hp)
        else:
            zs.zs_step(self.lay, self.G, self.state, self.p, full_flat,
                       grad_layout="slices", grad_stride=self.stride, step=t,
                       **hp)
        p16 = self.oracle_step(t, hp)
        if check:
            torch.cuda.synchronize()
            ma, m, v = read_state(self.lay_o, self.state)
            assert_parity(
                dict(master=ma, m=m, v=v, p=np16(self.p)),
                dict(master=self.om, m=self.omm, v=self.ov, p=p16),
                f"W={self.W} rank={self.rank} t={t} {self.layout}", exact)


def test_generator_device_matches_host():
    n = 1 << 20
    for base in (0, 12345, (1 << 33) + 7):
        t = dev_bf16(n)
        synth.dev_normal_bf16(t, 3, synth.TAG_GRAD, 2, 5, base, 1e-4)
        c = synth.cpu_normal_bf16(n, 3, synth.TAG_GRAD, 2, 5, base, 1e-4)
        assert np.array_equal(np16(t), c)
        f = dev_f32(n)
        synth.dev_normal_f32(f, 0, synth.TAG_V, 0, 0, base, 1e-8, absval=True)
        c = synth.cpu_normal_f32(n, 0, synth.TAG_V, 0, 0, base, 1e-8, True)
        assert np.array_equal(npf(f).view(np.uint32), c.view(np.uint32))


@pytest.mark.parametrize("W,cap", [(3, 3 * 256 * 37), (8, 25 << 20),
                                   (5, 0)])
def test_layout_conversions_match_the_oracle_mapping(W, cap):
    """zs_state_pack / zs_state_unpack / zs_grads_tile against the oracle's
    tile mapping, bit for bit, with ragged last tiles and NULL moments."""
    numels = [1000, 70000, 129, 20000, 9000]
    for rank in sorted({0, W - 1}):
        say(f"case conversions W={W} rank={rank} cap={cap}")
        lay_o = build_layout(numels, W, rank, cap)
        lay = zs.zs_layout_build(numels, W, rank, cap)
        n = lay_o.shard_numel
        ma = synth.cpu_normal_f32(n, 1, synth.TAG_MASTER, 0, 0, 0, 1.0)
        m = synth.cpu_normal_f32(n, 1, synth.TAG_M, 0, 0, 0, 1.0)
        v = synth.cpu_normal_f32(n, 1, synth.TAG_V, 0, 0, 0, 1.0, True)
        dma, dm, dv = (torch.from_numpy(x).cuda() for x in (ma, m, v))
        state = dev_f32(n_tiles(lay_o) * 3 * TILE)
        state.fill_(float("nan"))
        zs.zs_state_pack(lay, dma, dm, dv, state)
        want = to_tiled_state(lay_o, ma, m, v)
        assert np.array_equal(npf(state).view(np.uint32),
                              want.view(np.uint32))
        zs.zs_state_pack(lay, dma, None, None, state)
        zero = np.zeros(n, np.float32)
        assert np.array_equal(npf(state), to_tiled_state(lay_o, ma, zero,
                                                         zero))
        zs.zs_state_pack(lay, dma, dm, dv, state)
        outs = [dev_f32(n) for _ in range(3)]
        for o in outs:
            o.fill_(7.0)
        zs.zs_state_unpack(lay, state, *outs)
        for o, x in zip(outs, (ma, m, v)):
            assert np.array_equal(npf(o), x)
        zs.zs_state_unpack(lay, state, None, outs[1], None)
        G = np.stack([synth.cpu_bits16(n, 2, synth.TAG_SENTINEL, 0, s, 0)
                      for s in range(W)])
        stride = n + 40
        dG = torch.zeros((W, stride), dtype=torch.int16, device="cuda")
        dG[:, :n] = torch.from_numpy(G.view(np.int16)).cuda()
        Gt = dev_bf16(n_tiles(lay_o) * W * TILE)
        Gt.view(torch.int16).fill_(0x7fc0)
        zs.zs_grads_tile(lay, -1, dG, stride, Gt)
        assert np.array_equal(np16(Gt), to_tiled_grads(lay_o, G))
        # per bucket: the staging form of one bucket
        for b_id in (0, len(lay_o.buckets) - 1):
            b = lay_o.buckets[b_id]
            tb = -(-b.slice_numel // TILE)
            stg = torch.zeros((W, b.slice_numel + 8), dtype=torch.int16,
                              device="cuda")
            stg[:, :b.slice_numel] = dG[:, b.shard_off:b.shard_off
                                        + b.slice_numel]
            out = dev_bf16(tb * W * TILE)
            zs.zs_grads_tile(lay, b_id, stg, b.slice_numel + 8, out)
            full = to_tiled_grads(lay_o, G)
            lo = tile_offsets(lay_o)[b_id] * W * TILE
            assert np.array_equal(np16(out), full[lo:lo + tb * W * TILE])


@pytest.mark.parametrize("layout", LAYOUTS)
def test_tiny_three_steps(layout):
    w = wl.presets()["tiny"]
    say(f"case tiny W=4 rank 0 {layout}")
    c = Case(w.numels, w.world, w.rank, sigma=w.grad_sigma, layout=layout)
    for t in range(1, w.steps + 1):
        c.step(t)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_gpt2_thirteen_steps_and_flat_output(layout):
    """GPT-2-small-shaped, W=8, rank 0: ten warm-up steps then three more,
    compared after every step; the bf16 result also lands in the flat
    all-gather buffer at this rank's positions and nowhere else."""
    w = wl.presets()["gpt2"]
    say(f"case gpt2 W=8 rank 0 {layout}")
    c = Case(w.numels, w.world, w.rank, sigma=w.grad_sigma, layout=layout)
    F = c.lay_o.flat_numel
    flat = dev_bf16(F)
    synth.dev_bits16(flat, 9, synth.TAG_SENTINEL, 0, 0, 0)
    sentinel = synth.cpu_bits16(F, 9, synth.TAG_SENTINEL, 0, 0, 0)
    for t in range(1, w.warm_steps + w.steps + 1):
        c.step(t, full_flat=flat)
    torch.cuda.synchronize()
    ref = sentinel.copy()
    pack_flat(c.lay_o, c.op, ref)
    assert np.array_equal(np16(flat), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 7, 8, 16, 32, 64, 100, 128])
def test_every_world_size(W, layout):
    """Each compiled world size and the runtime-W kernel, several buckets, a
    ragged last bucket, slices that are not whole tiles, a staging stride
    longer than the shard, warm moments."""
    rng = random.Random(W)
    numels = [rng.choice([7, 129, 1000, 4096, 33333, 65536])
              for _ in range(9)]
    cap = W * 256 * rng.choice([3, 17, 40, 70])
    for rank in sorted({0, W - 1}):
        say(f"case W={W} rank={rank} cap={cap} {layout}")
        c = Case(numels, W, rank, cap=cap, stride_pad=24,
                 warm=(1e-4, 1e-8), seed=W, layout=layout)
        for t in (1, 2, 3):
            c.step(t)


@pytest.mark.parametrize("seed", range(40))
def test_random_configurations(seed):
    """Seeded random points of the whole parameter space: W from 1 to 128,
    any rank, tensor sizes around every alignment and tile boundary,
    alignment 16 B to 4 KiB, bucket caps from one unit up (or one bucket),
    the flat or whole-tensor layout, tiled or plain gradients with a padded
    stride, the mixed-precision or pure-bf16 step, cold or warm moments;
    two steps, bit for bit against the oracle."""
    rng = random.Random(4242 + seed)
    W = rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32, 48, 64, 100,
                    128])
    numels = [rng.choice([1, 7, 8, 127, 128, 129, 1000, 4095, 4096, 8191,
                          8193, 33333, 65536, 70001])
              for _ in range(rng.randint(1, 14))]
    tensors = rng.random() < 0.3
    align = rng.choice([16, 64, 256, 4096])
    cap = rng.choice([0, W * align * rng.randint(1, 40)])
    rank = rng.randrange(W)
    layout = rng.choice(LAYOUTS)
    pure = rng.random() < 0.3
    say(f"case random seed={seed} W={W} rank={rank} tensors={tensors} "
        f"align={align} cap={cap} {layout} pure={pure}")
    lay_o = (build_tensor_layout(numels, W, rank, align) if tensors
             else build_layout(numels, W, rank, cap, align))
    if lay_o.shard_numel == 0:          # a rank that owns nothing
        lay = (zs.zs_layout_build_tensors(numels, W, rank, align) if tensors
               else zs.zs_layout_build(numels, W, rank, cap, align))
        zs.zs_step(lay, dev_bf16(8), dev_f32(8), dev_bf16(8), None,
                   grad_layout=layout, grad_stride=8, step=1, **HP)
        return
    if pure:
        run_pure_bf16(numels, W, rank, cap, layout, rng.random() < 0.5,
                      (1, 2), tensors=tensors, align=align)
    else:
        c = Case(numels, W, rank, cap=cap, align=align,
                 stride_pad=rng.choice([0, 8, 24]),
                 warm=rng.choice([None, (1e-4, 1e-8)]), seed=seed,
                 layout=layout, tensors=tensors)
        for t in (1, 2):
            c.step(t)


HP_CASES = [
    ("lr 0", dict(HP, lr=0.0), (1, 2)),
    ("betas 0", dict(HP, beta1=0.0, beta2=0.0), (1, 2, 3)),
    ("no decay", dict(HP, weight_decay=0.0), (1, 2)),
    ("eps 1", dict(HP, eps=1.0), (1, 2)),
    ("large lr and decay", dict(HP, lr=1e-2, weight_decay=1.0), (1, 2)),
    ("late steps", HP, (1, 1000, 100000)),
    ("betas 0.999", dict(HP, beta1=0.999, beta2=0.999), (1, 7)),
]


@pytest.mark.parametrize("name,hp,steps", HP_CASES,
                         ids=[c[0] for c in HP_CASES])
def test_hyperparameter_edge_cases(name, hp, steps):
    """Degenerate and extreme hyper-parameters (lr = 0, betas 0 and 0.999,
    no decay, eps 1, large lr and decay, step counts up to 1e5 where the
    bias corrections reach 1) through the compiled-W and runtime-W kernels,
    bit for bit against the oracle."""
    for W in (8, 5):
        rng = random.Random(W)
        numels = [rng.choice([7, 129, 1000, 4096, 33333]) for _ in range(6)]
        say(f"case hp {name} W={W}")
        c = Case(numels, W, W - 1, cap=W * 256 * 17, warm=(1e-4, 1e-8),
                 seed=W, layout="tiled")
        for t in steps:
            c.step(t, hp=hp)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W,tiles", [(2, 300), (2, 4200), (16, 4100),
                                     (32, 4100), (64, 4100), (5, 4100),
                                     (5, 1100), (20, 1100), (12, 4100),
                                     (20, 4100), (33, 4100)])
def test_launch_shapes(W, tiles, layout):
    """Each work shape of the step: at a compiled W one-wave workgroups
    loading all W slices at once, in launches of fewer and of 4096 or more
    tiles (plain slice rows at W >= 32: Deep); at runtime W one-wave
    workgroups batching 8, 16 or 32 slices (below 4096 tiles only above
    W = 8, else Small; plain slice rows above W = 8: Small below 4096
    tiles, 4-slice batches below W = 32, 512-thread workgroups above); one
    bucket per launch, a ragged last tile."""
    n_rank = tiles * TILE - 4096            # the last tile half full
    numels = [W * n_rank - 1000, 1000]
    say(f"case shape W={W} tiles={tiles} {layout}")
    c = Case(numels, W, W - 1, cap=0, layout=layout)
    assert n_tiles(c.lay_o) == tiles
    for t in (1, 2):
        c.step(t)


def test_step_without_residency_cap():
    """zs_set_residency_cap(False): the same launches without the LDS
    reservation (only the dispatch differs), bit for bit against the oracle
    in a capped large launch, a capped small one and a runtime-W one."""
    prev = zs.zs_set_residency_cap(False)
    try:
        for W, tiles in ((8, 4100), (16, 300), (12, 4100)):
            n_rank = tiles * TILE - 4096
            say(f"case no residency cap W={W} tiles={tiles}")
            c = Case([W * n_rank], W, W - 1, cap=0, layout="tiled")
            for t in (1, 2):
                c.step(t)
    finally:
        zs.zs_set_residency_cap(prev)
    assert zs.zs_set_residency_cap(True) is True


@pytest.mark.parametrize("W,tiles,layout", [
    (3, 10, "tiled"), (8, 10, "slices"), (8, 4100, "tiled"),
    (5, 4100, "tiled"), (32, 4100, "tiled"), (64, 300, "tiled"),
    (64, 300, "slices")])
def test_sum_order_is_rank_order(W, tiles, layout):
    """Gradients where fp32 rounding exposes the order of the sum: every
    element's W slices hold one 1.0 at a position that varies with the
    element and 2^-24 everywhere else (half an ulp of 1.0, so each one
    added after the 1.0 ties back to it, while the ones before it add up
    exactly).  Every work shape, compiled and runtime W; bit for bit
    against the oracle, whose order is pinned on the same values."""
    n_rank = tiles * TILE - 4096            # the last tile half full
    numels = [W * n_rank]
    lay_o = build_layout(numels, W, W - 1, 0)
    lay = zs.zs_layout_build(numels, W, W - 1, 0)
    n = lay_o.shard_numel
    assert n_tiles(lay_o) == tiles
    say(f"case sum order W={W} tiles={tiles} {layout}")
    i = np.arange(n, dtype=np.int64)
    pos = (i * 7 + i // 13) % W
    G = np.full((W, n), 0x3380, np.uint16)
    G[pos, i] = 0x3F80
    state = dev_state(lay, lay_o, 0.02)
    om, omm, ov = read_state(lay_o, state)
    Gd = torch.from_numpy(G.view(np.int16)).cuda()
    if layout == "tiled":
        Gt = dev_bf16(n_tiles(lay_o) * W * TILE)
        zs.zs_grads_tile(lay, -1, Gd, n, Gt)
    p = dev_bf16(n)
    if layout == "tiled":
        zs.zs_step(lay, Gt, state, p, None, grad_layout="tiled", step=1,
                   **HP)
    else:
        zs.zs_step(lay, Gd, state, p, None, grad_stride=n, step=1, **HP)
    p16 = O.step(G, om, omm, ov, OHP, 1)
    torch.cuda.synchronize()
    gm, m1, v1 = read_state(lay_o, state)
    assert np.array_equal(gm.view(np.uint32), om.view(np.uint32))
    assert np.array_equal(m1.view(np.uint32), omm.view(np.uint32))
    assert np.array_equal(v1.view(np.uint32), ov.view(np.uint32))
    assert np.array_equal(np16(p), p16)
    # the order is visible in these values: the gradient means differ
    # between elements whose 1.0 sits at different positions
    g = O.reduce_mean(np.ascontiguousarray(G[:, :2 * W]))
    assert len(set(g.tolist())) > 1


@pytest.mark.parametrize("W,tiles", [(8, 4100), (5, 4100), (32, 4100),
                                     (64, 300)])
def test_pure_bf16_sum_order_is_rank_order(W, tiles):
    """The same order-exposing gradients through the pure-bf16 step's work
    shapes (its own 256-thread shape at W < 32, Deep, Small); parameter
    shard, bit for bit against the oracle."""
    n_rank = tiles * TILE - 4096
    numels = [W * n_rank]
    lay_o = build_layout(numels, W, W - 1, 0)
    lay = zs.zs_layout_build(numels, W, W - 1, 0)
    n = lay_o.shard_numel
    say(f"case bf16 sum order W={W} tiles={tiles}")
    i = np.arange(n, dtype=np.int64)
    G = np.full((W, n), 0x3380, np.uint16)
    G[(i * 7 + i // 13) % W, i] = 0x3F80
    om, omm, ov = S.cpu_state(0, n, 0.02, W, (), (1e-4, 1e-8))
    p16 = O.bf16_round(om)
    m_d, v_d = (torch.from_numpy(x.copy()).cuda() for x in (omm, ov))
    state = dev_f32(n_tiles(lay_o) * 2 * TILE)
    zs.zs_state_mv_pack(lay, m_d, v_d, state)
    params = torch.from_numpy(p16.view(np.int16).copy()).cuda()
    Gt = dev_bf16(n_tiles(lay_o) * W * TILE)
    zs.zs_grads_tile(lay, -1, torch.from_numpy(G.view(np.int16)).cuda(), n,
                     Gt)
    zs.zs_step_bf16(lay, Gt, state, params, params_flat=False,
                    grad_layout="tiled", step=1, **HP)
    O.step_bf16(G, p16, omm, ov, OHP, 1)
    torch.cuda.synchronize()
    m_g, v_g = from_tiled_rows(lay_o, npf(state), 2)
    assert np.array_equal(np16(params), p16)
    assert np.array_equal(m_g.view(np.uint32), omm.view(np.uint32))
    assert np.array_equal(v_g.view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("W", [3, 8])
def test_all_ranks_reassemble_to_the_unsharded_step(W):
    """all-reduce = reduce-scatter + all-gather on the GPU: every rank steps
    its own shard into one shared flat buffer; the flat buffer equals the
    oracle's step on the whole mean gradient, bit for bit."""
    numels = [5000, 7, 129, 70000, 300, 2047]
    cap = W * 256 * 20
    lay0 = build_layout(numels, W, 0, cap)
    F = lay0.flat_numel
    pad = np.ones(F, bool)
    for s0, n in zip(lay0.tensor_flat_off, numels):
        pad[s0:s0 + n] = False
    # the full local gradient of every source rank and the full master
    fullG = [np.zeros((W, F), np.uint16) for _ in range(2)]
    for t in (1, 2):
        for s in range(W):
            fullG[t - 1][s] = synth.cpu_normal_bf16(F, 0, synth.TAG_GRAD, t,
                                                    s, 0, 1e-3)
        fullG[t - 1][:, pad] = 0
    full_master = synth.cpu_normal_f32(F, 0, synth.TAG_MASTER, 0, 0, 0, 0.02)
    full_master[pad] = 0
    flat = dev_bf16(F)
    flat.view(torch.int16).fill_(0x7fc0)
    for r in range(W):
        say(f"case all-ranks W={W} rank={r}")
        lay_o = build_layout(numels, W, r, cap)
        lay = zs.zs_layout_build(numels, W, r, cap)
        idx = np.concatenate([np.arange(b.flat_off + r * b.slice_numel,
                                        b.flat_off + (r + 1) * b.slice_numel)
                              for b in lay_o.buckets])
        n = idx.size
        master = torch.from_numpy(full_master[idx].copy()).cuda()
        state = dev_f32(n_tiles(lay_o) * 3 * TILE)
        zs.zs_state_pack(lay, master, None, None, state)
        for t in (1, 2):
            G = torch.from_numpy(np.ascontiguousarray(
                fullG[t - 1][:, idx]).view(np.int16)).cuda()
            zs.zs_step(lay, G, state, None, flat, grad_stride=n, step=t,
                       **HP)
        torch.cuda.synchronize()
    # oracle: the whole mean gradient, one unsharded update
    om = full_master.copy()
    omm = np.zeros(F, np.float32)
    ov = np.zeros(F, np.float32)
    for t in (1, 2):
        acc = O.bf16_to_f32(fullG[t - 1][0]).copy()
        for s in range(1, W):
            acc = acc + O.bf16_to_f32(fullG[t - 1][s])
        p16 = O.adamw(acc / np.float32(W), om, omm, ov, OHP, t)
    assert np.array_equal(np16(flat), p16)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_bucket_steps_in_any_order_match_the_oracle(layout):
    """ZeRO-2 streaming on a second stream: buckets arrive in reverse order
    into a ring of S staging slots on an upload stream, each stepped by
    zs_bucket_step on a step stream once its copy has landed and before its
    slot is reused; after two steps the state and the bf16 shard equal the
    oracle's step of the whole shard, bit for bit."""
    w = wl.presets()["gpt2"]
    W = w.world
    ref = Case(w.numels, W, 0, sigma=w.grad_sigma, gpu=False)
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    for t in (1, 2):
        ref.oracle_step(t)
    slice_max = max(b.slice_numel for b in lay_o.buckets)
    tiles_max = -(-slice_max // TILE)
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    for slots in (1, 2, 3):
        say(f"case streaming slots={slots} {layout}")
        state = ref.dev_state()
        p = dev_bf16(n)
        if layout == "tiled":
            staging = [dev_bf16(tiles_max * W * TILE) for _ in range(slots)]
        else:
            staging = [torch.empty((W, slice_max), dtype=torch.bfloat16,
                                   device="cuda") for _ in range(slots)]
        up = torch.cuda.Stream()
        st = torch.cuda.Stream()
        done = [None] * slots
        order = list(range(len(lay_o.buckets)))[::-1]
        for t in (1, 2):
            ref.dev_grads(full, t)
            pool = [dev_tiled_bucket(full, lay_o, b_id) if layout == "tiled"
                    else None for b_id in range(len(lay_o.buckets))]
            torch.cuda.synchronize()
            for k, b_id in enumerate(order):
                b = lay_o.buckets[b_id]
                slot = k % slots
                with torch.cuda.stream(up):
                    if done[slot] is not None:
                        up.wait_event(done[slot])
                    if layout == "tiled":
                        staging[slot][:pool[b_id].numel()].copy_(pool[b_id])
                    else:
                        staging[slot][:, :b.slice_numel].copy_(
                            full[:, b.shard_off:b.shard_off + b.slice_numel])
                    landed = torch.cuda.Event()
                    landed.record(up)
                st.wait_event(landed)
                zs.zs_bucket_step(lay, b_id, staging[slot], state, p, None,
                                  grad_layout=layout, grad_stride=slice_max,
                                  step=t, stream=st, **HP)
                ev = torch.cuda.Event()
                ev.record(st)
                done[slot] = ev
            torch.cuda.synchronize()
        ref.check(state, f"streaming slots={slots} {layout}", p=p)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W,cap,groups", [
    (8, 25 << 20, [3, 1, 4, 2]),                 # GPT-2-shaped, 10 buckets
    (4, 4 * 256 * 8, [16, 16, 7, 1, 5]),         # 45 small buckets
    (12, 12 * 256 * 8, [6, 1, 5, 3]),            # runtime W, 15 buckets
])
def test_bucket_groups_match_the_oracle(W, cap, groups, layout):
    """zs_buckets_step over groups of buckets in a shuffled order, each
    bucket from its own staging buffer, the last rank (which holds the
    padding); after each of two steps the state, the bf16 shard and the
    flat buffer equal the oracle's, bit for bit."""
    numels = wl.gpt2_small() if W == 8 else [50000, 7, 129, 90000, 40000]
    ref = Case(numels, W, W - 1, cap=cap, gpu=False)
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    assert sum(groups) == len(lay_o.buckets)
    assert ref.pad                       # the last rank holds the padding
    say(f"case groups W={W} buckets={len(lay_o.buckets)} {groups} {layout}")
    state = ref.dev_state()
    p = dev_bf16(n)
    F = lay_o.flat_numel
    flat = dev_bf16(F)
    synth.dev_bits16(flat, 6, synth.TAG_SENTINEL, 0, 0, 0)
    flat0 = synth.cpu_bits16(F, 6, synth.TAG_SENTINEL, 0, 0, 0)
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    order = list(range(len(lay_o.buckets)))
    random.Random(W).shuffle(order)
    for t in (1, 2):
        ref.oracle_step(t)
        ref.dev_grads(full, t)
        k = 0
        for gsize in groups:
            ids = order[k:k + gsize]
            k += gsize
            stride = max(lay_o.buckets[b].slice_numel for b in ids)
            stg = []
            for b_id in ids:
                b = lay_o.buckets[b_id]
                if layout == "tiled":
                    stg.append(dev_tiled_bucket(full, lay_o, b_id))
                else:
                    # one common stride for the group: pad every staging row
                    y = torch.full((W, stride), float("nan"),
                                   dtype=torch.bfloat16, device="cuda")
                    y[:, :b.slice_numel] = full[:, b.shard_off:b.shard_off
                                                + b.slice_numel]
                    stg.append(y)
            zs.zs_buckets_step(lay, ids, stg, state, p, flat,
                               grad_layout=layout, grad_stride=stride,
                               step=t, **HP)
        ref.check(state, f"groups W={W} t={t} {layout}", p=p, flat=flat,
                  flat_before=flat0)


def run_plain(ref, layout, steps, stride_pad=8):
    """zs_step_plain on the case's shard (three plain fp32 arrays, the bf16
    shard and a sentinel-filled flat buffer) for the given steps, each
    checked against the oracle's arrays, bit for bit."""
    lay, lay_o, n, W = ref.lay, ref.lay_o, ref.n, ref.W
    master, m, v = dev_f32(n), dev_f32(n), dev_f32(n)
    S.dev_state(master, m, v, 0.02, ref.seed, ref.pad, ref.warm)
    p = dev_bf16(n)
    F = lay_o.flat_numel
    flat = dev_bf16(F)
    synth.dev_bits16(flat, 8, synth.TAG_SENTINEL, 0, 0, 0)
    flat0 = synth.cpu_bits16(F, 8, synth.TAG_SENTINEL, 0, 0, 0)
    G = torch.empty((W, n + stride_pad), dtype=torch.bfloat16, device="cuda")
    Gt = dev_bf16(max(n_tiles(lay_o) * W * TILE, 8))
    offs = tile_offsets(lay_o)
    for t in steps:
        ref.oracle_step(t)
        ref.dev_grads(G, t)
        if layout == "tiled":
            for b_id, t0 in enumerate(offs):
                x = dev_tiled_bucket(G, lay_o, b_id)
                Gt[t0 * W * TILE:t0 * W * TILE + x.numel()] = x
            zs.zs_step_plain(lay, Gt, master, m, v, p, flat,
                             grad_layout="tiled", step=t, **HP)
        else:
            zs.zs_step_plain(lay, G, master, m, v, p, flat,
                             grad_layout="slices", grad_stride=n + stride_pad,
                             step=t, **HP)
        torch.cuda.synchronize()
        where = f"plain W={W} rank={ref.rank} t={t} {layout}"
        assert_parity(dict(master=npf(master), m=npf(m), v=npf(v),
                           p=np16(p)),
                      dict(master=ref.om, m=ref.omm, v=ref.ov, p=ref.op),
                      where)
        want = flat0.copy()
        pack_flat(lay_o, ref.op, want)
        assert np.array_equal(np16(flat), want), f"{where}: flat buffer"


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W,tensors", [(1, False), (3, False), (8, False),
                                       (64, False), (100, False), (3, True),
                                       (8, True)])
def test_plain_state_step(W, tensors, layout):
    """zs_step_plain, the step on three plain fp32 arrays (master, m, v)
    instead of the tiled state: compiled and runtime W, several buckets with
    ragged slices (or the owned tensors of the whole-tensor layout), warm
    moments, three steps; the state, the bf16 shard and the flat buffer
    against the oracle, bit for bit."""
    rng = random.Random(500 + W)
    if tensors:
        numels, cap = TENSOR_LIST, None
    else:
        numels = [rng.choice([7, 129, 1000, 4096, 33333, 65536])
                  for _ in range(9)]
        cap = W * 256 * rng.choice([3, 17, 40])
    say(f"case plain state W={W} tensors={tensors} {layout}")
    ref = Case(numels, W, W - 1, cap=cap if cap else 25 << 20,
               tensors=tensors, warm=(1e-4, 1e-8), seed=W, gpu=False)
    run_plain(ref, layout, (1, 2, 3))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W,tiles", [(8, 4100), (5, 4100), (20, 4100),
                                     (32, 4100), (48, 4100)])
def test_plain_state_launch_shapes(W, tiles, layout):
    """zs_step_plain in the work shapes of large launches (one-wave at
    compiled and runtime W; on plain slices Deep at W = 32, Wave at W = 20,
    Wide at W = 48): one bucket, a ragged last tile; two steps against the
    oracle."""
    n_rank = tiles * TILE - 4096
    say(f"case plain state shape W={W} tiles={tiles} {layout}")
    ref = Case([W * n_rank], W, W - 1, cap=0, seed=W, gpu=False)
    assert n_tiles(ref.lay_o) == tiles
    run_plain(ref, layout, (1, 2), stride_pad=0)


def test_pack_flat_and_per_tensor():
    w = wl.presets()["gpt2"]
    for rank in (0, 5, 7):
        say(f"case pack rank={rank}")
        lay_o = build_layout(w.numels, w.world, rank)
        lay = zs.zs_layout_build(w.numels, w.world, rank)
        n = lay_o.shard_numel
        shard = dev_bf16(n)
        synth.dev_bits16(shard, rank, synth.TAG_SENTINEL, 1, 0, 0)
        host_shard = synth.cpu_bits16(n, rank, synth.TAG_SENTINEL, 1, 0, 0)
        F = lay_o.flat_numel
        flat = dev_bf16(F)
        synth.dev_bits16(flat, 2, synth.TAG_SENTINEL, 2, 0, 0)
        ref_flat = synth.cpu_bits16(F, 2, synth.TAG_SENTINEL, 2, 0, 0)
        # per-tensor storage; odd element offsets make some pointers
        # unaligned so both copy paths run
        tensors = []
        for k, numel in enumerate(w.numels):
            off = 1 if k % 3 == 1 else 0
            base = dev_bf16(numel + off)
            base.view(torch.int16).fill_(k)
            tensors.append(base[off:])
        ptrs = torch.tensor([t.data_ptr() for t in tensors],
                            dtype=torch.int64, device="cuda")
        chunks = zs.zs_layout_chunks(lay)
        raw = np.frombuffer(zs.chunks_bytes(chunks), np.uint8).copy()
        dchunks = torch.from_numpy(raw).cuda()
        zs.zs_pack(lay, shard, flat, dchunks, len(chunks), ptrs)
        torch.cuda.synchronize()
        pack_flat(lay_o, host_shard, ref_flat)
        assert np.array_equal(np16(flat), ref_flat)
        ref_t = [np.full(nm, k, np.uint16) for k, nm in enumerate(w.numels)]
        pack_tensors(lay_o, host_shard, ref_t)
        for t_, r_ in zip(tensors, ref_t):
            assert np.array_equal(np16(t_), r_)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_nan_is_local_and_padding_stays_zero(layout):
    numels = [1000, 3]          # rank 2 of 4: two tensors and two pads
    lay_o = build_layout(numels, 4, 2, 0)
    lay = zs.zs_layout_build(numels, 4, 2, 0)
    n = lay_o.shard_numel
    pad = S.padding_runs(n, lay_o.chunks)
    assert pad
    G = torch.zeros((4, n), dtype=torch.bfloat16, device="cuda")
    S.dev_grads(G, 4, n, 1, 1e-3, pad=pad)
    G.view(torch.int16)[2, 5] = 0x7fc0
    state = dev_state(lay, lay_o, 0.02, pad=pad)
    p = dev_bf16(n)
    Gt = dev_bf16(n_tiles(lay_o) * 4 * TILE)
    zs.zs_grads_tile(lay, -1, G, n, Gt)
    for t in (1, 2):
        if layout == "tiled":
            zs.zs_step(lay, Gt, state, p, None, grad_layout="tiled", step=t,
                       **HP)
        else:
            zs.zs_step(lay, G, state, p, None, grad_stride=n, step=t, **HP)
    torch.cuda.synchronize()
    mm, m1, v1 = read_state(lay_o, state)
    assert np.isnan(mm[5]) and np.isfinite(np.delete(mm, 5)).all()
    for s0, e0 in pad:
        assert not mm[s0:e0].view(np.uint32).any()
        assert not m1[s0:e0].view(np.uint32).any()
        assert not v1[s0:e0].view(np.uint32).any()
        assert not np16(p)[s0:e0].any()


def sample_windows(lay_o, per_bucket=4096, chunk_side=512, n_even=64,
                   even_span=1 << 20, n_random=8, span=1 << 16, seed=0):
    """Shard windows (the step is elementwise, so each window checks on its
    own): the first and last per_bucket elements of every bucket slice,
    chunk_side elements on both sides of every chunk boundary, n_even
    evenly spaced windows of even_span elements, and random spans."""
    n = lay_o.shard_numel
    wins = []
    for b in lay_o.buckets:
        wins.append((b.shard_off, min(per_bucket, b.slice_numel)))
        e = b.shard_off + b.slice_numel
        wins.append((max(b.shard_off, e - per_bucket), min(per_bucket,
                                                           b.slice_numel)))
    for c in lay_o.chunks:
        a = max(0, c.shard_off - chunk_side) // 8 * 8
        wins.append((a, min(2 * chunk_side, n - a)))
    for i in range(n_even):
        a = (n - even_span) * i // max(1, n_even - 1) // 8 * 8
        wins.append((max(0, a), min(even_span, n)))
    rng = random.Random(seed)
    for _ in range(n_random):
        a = rng.randrange(0, max(1, n - span)) // 8 * 8
        wins.append((a, min(span, n - a)))
    return wins


@pytest.mark.parametrize("name,tensors", [("llama8b", False),
                                          ("dense7b", False),
                                          ("llama8b", True)])
def test_full_size_sampled(name, tensors):
    """The full Llama-3-8B-shaped (W=8) and 7B-shaped (W=64) rank-0 shards,
    in the launch configuration the benchmark times (tiled gradients, tiled
    state, bf16 result straight into the flat all-gather buffer), in the
    flat layout and (8B) the whole-tensor assignment; sampled windows
    against the oracle after each step."""
    w = wl.presets()[name]
    if tensors:
        lay_o = build_tensor_layout(w.numels, w.world, 0)
        lay = zs.zs_layout_build_tensors(w.numels, w.world, 0)
    else:
        lay_o = build_layout(w.numels, w.world, 0)
        lay = zs.zs_layout_build(w.numels, w.world, 0)
    n, W = lay_o.shard_numel, w.world
    say(f"case full-size {name}{' whole tensors' if tensors else ''}: "
        f"W={W} shard={n}")
    state = dev_state(lay, lay_o, w.master_sigma)
    G = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    Gt = dev_bf16(n_tiles(lay_o) * W * TILE)
    flat = dev_bf16(lay_o.flat_numel)
    flat.view(torch.int16).fill_(0x7fc0)
    # W = 64 makes each window 8 times dearer to generate on the host
    wins = sample_windows(lay_o, n_even=64 if W <= 8 else 16)
    ref = [S.cpu_state(a, k, w.master_sigma) for a, k in wins]
    slot = tile_slot(lay_o)
    st3 = state.view(n_tiles(lay_o), 3, TILE)
    for t in (1, 2):
        S.dev_grads(G, W, n, t, w.grad_sigma)
        zs.zs_grads_tile(lay, -1, G, n, Gt)
        zs.zs_step(lay, Gt, state, None, flat, grad_layout="tiled", step=t,
                   **HP)
        torch.cuda.synchronize()
        for (a, k), st in zip(wins, ref):
            Gc = S.cpu_grads(W, a, k, t, w.grad_sigma)
            p16 = O.step(Gc, *st, OHP, t)
            sl = torch.from_numpy(slot[a:a + k]).cuda()
            ti, pi = sl // TILE, sl % TILE
            got = [npf(st3[ti, row, pi]) for row in range(3)]
            fpos = []
            for b in lay_o.buckets:   # flat position of each shard element
                lo, hi = max(a, b.shard_off), min(a + k, b.shard_off
                                                  + b.slice_numel)
                if hi > lo:
                    fpos.append((lo - a, hi - a, b.flat_off + (lo
                                                               - b.shard_off)))
            got_p = np.empty(k, np.uint16)
            for s0, e0, f0 in fpos:
                got_p[s0:e0] = np16(flat[f0:f0 + (e0 - s0)])
            assert_parity(
                dict(master=got[0], m=got[1], v=got[2], p=got_p),
                dict(master=st[0], m=st[1], v=st[2], p=p16),
                f"{name} t={t} window {a}+{k}")
    # rank 0 writes nothing outside its slices (its tensors)
    if tensors:
        others = [t for t, r in enumerate(lay_o.owner) if r != 0]
        spots = [lay_o.tensor_flat_off[t] for t in others[:3] + others[-2:]]
    else:
        spots = [b.flat_off + b.slice_numel
                 for b in lay_o.buckets[:3] + lay_o.buckets[-2:]]
    for f0 in spots:
        assert np.all(np16(flat[f0:f0 + 4096]) == 0x7fc0), f0


def test_streaming_70b_sampled_beyond_2_32():
    """The Llama-3-70B-shaped W=16 rank-0 shard at full size (4.41e9
    elements; shard, tile, state and flat offsets beyond 2^32), in the
    launch configuration the streaming benchmark times: a group of 16
    buckets (from the start, the thirds, the middle and the end of the
    shard), each from its own tiled staging buffer, stepped twice by one
    zs_buckets_step call that writes the bf16 result into the 141 GB flat
    buffer (and the shard); windows at both ends of every stepped slice
    against the oracle."""
    w = wl.presets()["llama70b"]
    lay_o = build_layout(w.numels, w.world, 0)
    lay = zs.zs_layout_build(w.numels, w.world, 0)
    n, W, nb = lay_o.shard_numel, w.world, len(lay_o.buckets)
    assert n > 2 ** 32
    say(f"case 70b sampled: W={W} shard={n} buckets={nb}")
    state = dev_f32(n_tiles(lay_o) * 3 * TILE)
    master = dev_f32(n)
    synth.dev_normal_f32(master, 0, synth.TAG_MASTER, 0, 0, 0,
                         w.master_sigma)
    zs.zs_state_pack(lay, master, None, None, state)
    torch.cuda.synchronize()
    del master
    torch.cuda.empty_cache()
    p = dev_bf16(n)
    flat = dev_bf16(lay_o.flat_numel)
    ids = [0, 1, 2, 3, nb // 3, nb // 3 + 1, nb // 2, nb // 2 + 1,
           2 * nb // 3, 2 * nb // 3 + 1, nb - 6, nb - 5, nb - 4, nb - 3,
           nb - 2, nb - 1]
    assert len(set(ids)) == zs.ZS_MAX_GROUP == 16
    assert lay_o.buckets[nb - 1].shard_off > 2 ** 32
    smax = max(lay_o.buckets[b].slice_numel for b in ids)
    tmp = torch.empty((W, smax), dtype=torch.bfloat16, device="cuda")
    stg = [dev_bf16(-(-smax // TILE) * W * TILE) for _ in ids]
    st3 = state.view(n_tiles(lay_o), 3, TILE)
    wins = []
    for b_id in ids:
        b = lay_o.buckets[b_id]
        for j0 in (0, b.slice_numel - 2048):
            wins.append((b_id, j0, 2048))
    ref = {x: S.cpu_state(lay_o.buckets[x[0]].shard_off + x[1], x[2],
                          w.master_sigma) for x in wins}
    for t in (1, 2):
        for b_id, buf in zip(ids, stg):
            b = lay_o.buckets[b_id]
            for s in range(W):
                synth.dev_normal_bf16(tmp[s, :b.slice_numel], 0,
                                      synth.TAG_GRAD, t, s, b.shard_off,
                                      w.grad_sigma)
            zs.zs_grads_tile(lay, b_id, tmp, smax, buf)
        zs.zs_buckets_step(lay, ids, stg, state, p, flat,
                           grad_layout="tiled", step=t, **HP)
        torch.cuda.synchronize()
        for (b_id, j0, k) in wins:
            b = lay_o.buckets[b_id]
            a = b.shard_off + j0
            st = ref[(b_id, j0, k)]
            p16 = O.step(S.cpu_grads(W, a, k, t, w.grad_sigma), *st, OHP, t)
            sl = torch.from_numpy(tile_slot_range(lay_o, b_id, j0, k)).cuda()
            ti, pi = sl // TILE, sl % TILE
            got = [npf(st3[ti, row, pi]) for row in range(3)]
            assert_parity(
                dict(master=got[0], m=got[1], v=got[2],
                     p=np16(p[a:a + k])),
                dict(master=st[0], m=st[1], v=st[2], p=p16),
                f"70b t={t} bucket {b_id} window {j0}+{k}")
            f0 = b.flat_off + j0                # rank 0's slice position
            assert np.array_equal(np16(flat[f0:f0 + k]), p16)


@pytest.mark.parametrize("W,cap", [(1, 25 << 20), (3, 3 * 256 * 37),
                                   (8, 8 * 256 * 11), (64, 0)])
def test_gather_matches_the_oracle(W, cap):
    """zs_gather (ZeRO-3 / FSDP materialisation) against the oracle, bit for
    bit: the whole flat buffer, every tensor, runs of tensors, random
    windows with a ragged end; nothing written past the range."""
    numels = [1000, 70000, 7, 129, 20000, 9000, 3]
    lay_o = build_layout(numels, W, 0, cap)
    lay = zs.zs_layout_build(numels, W, 0, cap)
    n, F = lay_o.shard_numel, lay_o.flat_numel
    say(f"case gather W={W} cap={cap} flat={F}")
    host = [synth.cpu_bits16(n, 4, synth.TAG_SENTINEL, 0, r, 0)
            for r in range(W)]
    dev = [torch.from_numpy(h.view(np.int16)).cuda() for h in host]
    out = torch.empty(F + 64, dtype=torch.int16, device="cuda")
    rng = random.Random(W)
    offs = lay_o.tensor_flat_off
    ranges = [(0, F)] + [(o, o + k) for o, k in zip(offs, numels)]
    ranges += [(offs[1], offs[4] + numels[4]), (offs[2], offs[6] + 3)]
    for _ in range(6):
        lo = rng.randrange(0, F) // 8 * 8
        ranges.append((lo, rng.randrange(lo, F + 1)))
    for lo, hi in ranges:
        out.fill_(0x5a5a)
        zs.zs_gather(lay, dev, lo, hi, out)
        got = np16(out)
        assert np.array_equal(got[:hi - lo],
                              gather(numels, W, host, lo, hi, cap)), (lo, hi)
        assert np.all(got[hi - lo:] == 0x5a5a), (lo, hi)


def test_gather_across_launches():
    """A gather whose range spans more buckets than one launch holds (W = 64,
    8192-element buckets: 1023 buckets per launch): the first launch starts
    at the range's first rank row, the last ends at its last, the rows in
    between whole; against the oracle bit for bit, nothing written past the
    range."""
    W, cap = 64, 64 * 256
    numels = [3_000_000, 5_000_000, 700_001, 129, 40_000]
    lay_o = build_layout(numels, W, 0, cap)
    lay = zs.zs_layout_build(numels, W, 0, cap)
    n, F = lay_o.shard_numel, lay_o.flat_numel
    B = lay_o.buckets[0].numel
    per_launch = 65535 // W
    assert len(lay_o.buckets) > per_launch + 1
    say(f"case gather across launches W={W} buckets={len(lay_o.buckets)}")
    host = [synth.cpu_bits16(n, 5, synth.TAG_SENTINEL, 0, r, 0)
            for r in range(W)]
    dev = [torch.from_numpy(h.view(np.int16)).cuda() for h in host]
    full = gather(numels, W, host, 0, F, cap)
    out = torch.empty(F + 64, dtype=torch.int16, device="cuda")
    S = B // W
    edge = per_launch * B                       # first bucket of launch 2
    ranges = [(0, F), (8, F - 3), (edge - 5 * S + 40, edge + 3 * S + 17),
              (edge, edge + B), (edge - B + 2 * S, edge + 1),
              (S * 3 + 8, S * 5 - 1), (F - S - 800, F)]
    rng = random.Random(7)
    for _ in range(4):
        lo = rng.randrange(0, edge) // 8 * 8
        ranges.append((lo, rng.randrange(edge, F + 1)))
    for lo, hi in ranges:
        assert 0 <= lo < hi <= F and lo % 8 == 0, (lo, hi)
        out.fill_(0x5a5a)
        zs.zs_gather(lay, dev, lo, hi, out)
        got = np16(out)
        assert np.array_equal(got[:hi - lo], full[lo:hi]), (lo, hi)
        assert np.all(got[hi - lo:] == 0x5a5a), (lo, hi)


def test_gather_llama8b_layers_sampled():
    """Full-size Llama-3-8B-shaped W=8 layout: the embedding, a middle
    block and the final norm + lm_head gathered from 8 resident shards;
    sampled windows against the oracle's ownership runs."""
    w = wl.presets()["llama8b"]
    lay_o = build_layout(w.numels, w.world, 0)
    lay = zs.zs_layout_build(w.numels, w.world, 0)
    n, W = lay_o.shard_numel, w.world
    say(f"case gather llama8b: W={W} shard={n}")
    dev = []
    for r in range(W):
        t = dev_bf16(n)
        synth.dev_bits16(t, 5, synth.TAG_SENTINEL, 0, r, 0)
        dev.append(t)
    offs, nm = lay_o.tensor_flat_off, w.numels
    units = [(0, 0), (1 + 9 * 15, 9 + 9 * 15), (len(nm) - 2, len(nm) - 1)]
    rng = random.Random(8)
    for t0, t1 in units:
        lo, hi = offs[t0], offs[t1] + nm[t1]
        out = dev_bf16(hi - lo + 8)
        out.view(torch.int16).fill_(0x5a5a)
        zs.zs_gather(lay, dev, lo, hi, out)
        torch.cuda.synchronize()
        wins = [(lo, 4096), (hi - 4096, 4096)] + \
            [(lo + rng.randrange(0, hi - lo - 65536), 65536)
             for _ in range(8)]
        for a, k in wins:
            want = np.empty(k, np.uint16)
            for f0, m, r, s0 in owner_runs(lay_o, a, a + k):
                want[f0 - a:f0 - a + m] = synth.cpu_bits16(
                    m, 5, synth.TAG_SENTINEL, 0, r, s0)
            assert np.array_equal(np16(out[a - lo:a - lo + k]), want), \
                (t0, a, k)
        assert np.all(np16(out[hi - lo:]) == 0x5a5a)


@pytest.mark.parametrize("flat_params", [False, True])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W", [1, 3, 8, 16, 64, 100])
def test_pure_bf16_step(W, layout, flat_params):
    """zs_step_bf16 (no fp32 master, 12 B/param) against the oracle, bit for
    bit, three steps with warm moments; parameters as the bf16 shard or in
    place in the flat buffer (other ranks' positions untouched)."""
    rng = random.Random(100 + W)
    numels = [rng.choice([7, 129, 1000, 4096, 33333, 65536])
              for _ in range(9)]
    cap = W * 256 * rng.choice([3, 17, 40])
    say(f"case bf16 W={W} {layout} flat={flat_params}")
    run_pure_bf16(numels, W, W - 1, cap, layout, flat_params, (1, 2, 3))


@pytest.mark.parametrize("W,tiles", [(2, 300), (2, 4200), (8, 4100),
                                     (5, 4100), (12, 4100), (32, 4100),
                                     (33, 4100)])
def test_pure_bf16_launch_shapes(W, tiles):
    """Each work shape of the pure-bf16 step: one-wave workgroups at a
    compiled W (fewer and 4096 or more tiles), and at runtime W one-wave
    workgroups of 4-slice batches up to W = 8 and of 16- or 32-slice
    batches above;
    one bucket, a ragged last tile, parameters in place in the flat
    buffer, tiled gradients; bit for bit against the oracle."""
    n_rank = tiles * TILE - 4096            # the last tile half full
    numels = [W * n_rank - 1000, 1000]
    say(f"case bf16 shape W={W} tiles={tiles}")
    lay_o = run_pure_bf16(numels, W, W - 1, 0, "tiled", True, (1, 2))
    assert n_tiles(lay_o) == tiles


def run_pure_bf16(numels, W, rank, cap, layout, flat_params, steps,
                  tensors=False, align=256):
    """zs_step_bf16 on rank `rank`'s shard for the given steps, checked
    after each against the oracle, bit for bit; returns the oracle layout.
    tensors: the whole-tensor assignment instead of the flat layout."""
    if tensors:
        lay_o = build_tensor_layout(numels, W, rank, align)
        lay = zs.zs_layout_build_tensors(numels, W, rank, align)
    else:
        lay_o = build_layout(numels, W, rank, cap, align)
        lay = zs.zs_layout_build(numels, W, rank, cap, align)
    n, F = lay_o.shard_numel, lay_o.flat_numel
    pad = S.padding_runs(n, lay_o.chunks)
    om, omm, ov = S.cpu_state(0, n, 0.02, W, pad, (1e-4, 1e-8))
    p16 = O.bf16_round(om)
    m_d, v_d = (torch.from_numpy(x.copy()).cuda() for x in (omm, ov))
    state = dev_f32(n_tiles(lay_o) * 2 * TILE)
    state.fill_(float("nan"))
    zs.zs_state_mv_pack(lay, m_d, v_d, state)
    assert np.array_equal(npf(state), to_tiled_rows(lay_o, [omm, ov]))
    if flat_params:
        sentinel = synth.cpu_bits16(F, 7, synth.TAG_SENTINEL, 0, 0, 0)
        host_flat = sentinel.copy()
        pack_flat(lay_o, p16, host_flat)
        params = torch.from_numpy(host_flat.view(np.int16)).cuda()
    else:
        params = torch.from_numpy(p16.view(np.int16).copy()).cuda()
    G = torch.empty((W, n + 8), dtype=torch.bfloat16, device="cuda")
    Gt = dev_bf16(n_tiles(lay_o) * W * TILE)
    for t in steps:
        S.dev_grads(G, W, n, t, 1e-3, W, pad)
        if layout == "tiled":
            zs.zs_grads_tile(lay, -1, G, n + 8, Gt)
            zs.zs_step_bf16(lay, Gt, state, params, params_flat=flat_params,
                            grad_layout="tiled", step=t, **HP)
        else:
            zs.zs_step_bf16(lay, G, state, params, params_flat=flat_params,
                            grad_stride=n + 8, step=t, **HP)
        O.step_bf16(S.cpu_grads(W, 0, n, t, 1e-3, W, pad), p16, omm, ov,
                    OHP, t)
        torch.cuda.synchronize()
        m_g, v_g = from_tiled_rows(lay_o, npf(state), 2)
        if flat_params:
            want = sentinel.copy()
            pack_flat(lay_o, p16, want)
            got_p = np16(params)
        else:
            want, got_p = p16, np16(params)
        assert np.array_equal(got_p, want), f"params t={t}"
        assert np.array_equal(m_g.view(np.uint32), omm.view(np.uint32))
        assert np.array_equal(v_g.view(np.uint32), ov.view(np.uint32))
    outs = [dev_f32(n), dev_f32(n)]
    zs.zs_state_mv_unpack(lay, state, *outs)
    assert np.array_equal(npf(outs[0]), omm)
    assert np.array_equal(npf(outs[1]), ov)
    return lay_o


def test_pure_bf16_llama8b_flat_sampled():
    """Full-size Llama-3-8B-shaped W=8 rank-0 shard, pure bf16, tiled
    gradients, parameters updated in place in the flat buffer; sampled
    windows against the oracle after each of two steps."""
    w = wl.presets()["llama8b"]
    lay_o = build_layout(w.numels, w.world, 0)
    lay = zs.zs_layout_build(w.numels, w.world, 0)
    n, W = lay_o.shard_numel, w.world
    say(f"case bf16 full-size llama8b: W={W} shard={n}")
    state = dev_f32(n_tiles(lay_o) * 2 * TILE)
    zs.zs_state_mv_pack(lay, None, None, state)
    master = dev_f32(n)
    synth.dev_normal_f32(master, 0, synth.TAG_MASTER, 0, 0, 0,
                         w.master_sigma)
    shard16 = dev_bf16(n)
    flat = dev_bf16(lay_o.flat_numel)
    flat.view(torch.int16).fill_(0x7fc0)
    # the initial bf16 parameters: the master rounded on the host, per window
    wins = sample_windows(lay_o, n_random=8)
    G = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    Gt = dev_bf16(n_tiles(lay_o) * W * TILE)
    # round the device master to bf16 through the oracle's rule, window by
    # window, and place the whole shard with the pack (its own parity test)
    host_master = npf(master)
    del master
    shard16.copy_(torch.from_numpy(O.bf16_round(host_master).view(np.int16)
                                   ).view(torch.bfloat16).cuda())
    zs.zs_pack(lay, shard16, flat)
    ref = {}
    for a, k in wins:
        ref[(a, k)] = [O.bf16_round(host_master[a:a + k]),
                       np.zeros(k, np.float32), np.zeros(k, np.float32)]
    del host_master
    for t in (1, 2):
        S.dev_grads(G, W, n, t, w.grad_sigma)
        zs.zs_grads_tile(lay, -1, G, n, Gt)
        zs.zs_step_bf16(lay, Gt, state, flat, params_flat=True,
                        grad_layout="tiled", step=t, **HP)
        torch.cuda.synchronize()
        st2 = state.view(n_tiles(lay_o), 2, TILE)
        slot = None
        for (a, k), (p16, mm, vv) in ref.items():
            O.step_bf16(S.cpu_grads(W, a, k, t, w.grad_sigma), p16, mm, vv,
                        OHP, t)
            got_p = np.empty(k, np.uint16)
            for b in lay_o.buckets:
                lo, hi = max(a, b.shard_off), min(a + k, b.shard_off
                                                  + b.slice_numel)
                if hi > lo:
                    f0 = b.flat_off + (lo - b.shard_off)
                    got_p[lo - a:hi - a] = np16(flat[f0:f0 + hi - lo])
            assert np.array_equal(got_p, p16), f"t={t} window {a}+{k}"
            sl = []
            for b_id, b in enumerate(lay_o.buckets):
                lo, hi = max(a, b.shard_off), min(a + k, b.shard_off
                                                  + b.slice_numel)
                if hi > lo:
                    sl.append(tile_slot_range(lay_o, b_id, lo - b.shard_off,
                                              hi - lo))
            slot = torch.from_numpy(np.concatenate(sl)).cuda()
            ti, pi = slot // TILE, slot % TILE
            assert np.array_equal(npf(st2[ti, 0, pi]).view(np.uint32),
                                  mm.view(np.uint32))
            assert np.array_equal(npf(st2[ti, 1, pi]).view(np.uint32),
                                  vv.view(np.uint32))


@pytest.mark.parametrize("k", [2, 3, 4, 8])
def test_gradient_accumulation(k):
    """zs_accumulate over k micro-batches against the oracle, bit for bit;
    a length that ends inside a chunk; the last call writing over the
    last micro-batch's gradient (out aliasing grad); acc untouched by it."""
    n = 4096 * 5 + 12
    say(f"case accumulate k={k} n={n}")
    G = np.stack([synth.cpu_normal_bf16(n, k, synth.TAG_GRAD, j, 0, 0, 1.0)
                  for j in range(k)])
    G[0, :4] = [0x7fc0, 0xff80, 0x0001, 0x8000]     # NaN, -Inf, denormal, -0
    want = O.accumulate(G)
    dG = torch.from_numpy(G.view(np.int16)).cuda()
    acc = dev_f32(n)
    zs.zs_accumulate(zs.ZS_ACC_FIRST, acc, dG[0])
    for j in range(1, k - 1):
        zs.zs_accumulate(zs.ZS_ACC_ADD, acc, dG[j])
    before = acc.clone()
    zs.zs_accumulate(zs.ZS_ACC_LAST, acc, dG[k - 1], dG[k - 1], k=k)
    torch.cuda.synchronize()
    assert np.array_equal(np16(dG[k - 1]), want)
    assert torch.equal(acc.view(torch.int32), before.view(torch.int32))


def test_gradient_accumulation_llama8b_flat_sampled():
    """The benchmark's accumulation workload at full size: the Llama-3-8B-
    shaped flat gradient buffer (8.03e9 elements, offsets beyond 2^32),
    three micro-batches (first, add, last written over the last gradient);
    sampled windows at both ends, around 2^32 and 3 * 2^31 and at random
    against the oracle, bit for bit."""
    w = wl.presets()["llama8b"]
    n = build_layout(w.numels, w.world, 0).flat_numel
    k = 3
    say(f"case accumulate full-size llama8b: n={n} k={k}")
    G = [dev_bf16(n) for _ in range(k)]
    for j, g in enumerate(G):
        synth.dev_normal_bf16(g, 0, synth.TAG_GRAD, j, 0, 0, w.grad_sigma)
    acc = dev_f32(n)
    zs.zs_accumulate(zs.ZS_ACC_FIRST, acc, G[0])
    zs.zs_accumulate(zs.ZS_ACC_ADD, acc, G[1])
    zs.zs_accumulate(zs.ZS_ACC_LAST, acc, G[2], G[2], k=k)
    torch.cuda.synchronize()
    rng = random.Random(11)
    wins = [(0, 8192), (n - 8192, 8192), (2 ** 32 - 4096, 8192),
            (3 * 2 ** 31 - 4096, 8192)]
    assert all(a + m <= n for a, m in wins)
    wins += [(rng.randrange(0, n - 65536) // 8 * 8, 65536) for _ in range(8)]
    for a, m in wins:
        Gh = np.stack([synth.cpu_normal_bf16(m, 0, synth.TAG_GRAD, j, 0, a,
                                             w.grad_sigma)
                       for j in range(k)])
        assert np.array_equal(np16(G[k - 1][a:a + m]), O.accumulate(Gh)), a


def engine_case(numels, W, rank, cap=None, tensors=False, warm=None,
                sigma=1e-3, seed=0):
    """An oracle-only Case for the engine tests, with a sentinel-filled
    flat buffer on the device and its host copy."""
    ref = Case(numels, W, rank, cap=cap if cap is not None else 25 << 20,
               tensors=tensors, warm=warm, sigma=sigma, seed=seed, gpu=False)
    F = ref.lay_o.flat_numel
    flat = dev_bf16(F)
    synth.dev_bits16(flat, 4, synth.TAG_SENTINEL, 0, 0, 0)
    flat0 = synth.cpu_bits16(F, 4, synth.TAG_SENTINEL, 0, 0, 0)
    return ref, flat, flat0


def bucket_pool(ref, full, t, host=False):
    """Every bucket's step-t gradients in the tiled staging form, in device
    memory (or pinned host memory)."""
    ref.dev_grads(full, t)
    pool = [dev_tiled_bucket(full, ref.lay_o, b_id)
            for b_id in range(len(ref.lay_o.buckets))]
    if host:
        pool = [x.cpu().pin_memory() for x in pool]
    return pool


def slot_elems(lay_o, W):
    return max(-(-b.slice_numel // TILE) for b in lay_o.buckets) * W * TILE


@pytest.mark.parametrize("arrival,tensors,n_up", [
    ("device", False, 1), ("pinned host", False, 1), ("device", True, 1),
    ("pinned host", False, 4), ("device", True, 3)])
def test_stream_engine_matches_the_oracle(arrival, tensors, n_up):
    """The streaming engine (zs_stream_*): a rank's buckets (owned tensors
    in the whole-tensor layout) arrive one by one in a shuffled order, from
    device or pinned host memory, over one or several upload streams, into
    a ring of 2 x 3 staging slots; groups of 3 alternate over two step
    streams; after each of two steps the state, the shard and the flat
    buffer equal the oracle's, bit for bit.  A bucket arriving twice and a
    misaligned or short state are refused."""
    W, rank = 4, 1
    numels = [5000, 7, 129, 70000, 300, 2047, 40000, 9000]
    if tensors:
        numels = numels + TENSOR_LIST + [333, 4444, 55555, 6]
    ref, flat, flat0 = engine_case(numels, W, rank, cap=W * 256 * 9,
                                   tensors=tensors, warm=(1e-4, 1e-8))
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    nb = len(lay_o.buckets)
    assert nb > 4
    say(f"case stream engine W={W} buckets={nb} arrival={arrival} "
        f"tensors={tensors} upload streams={n_up}")
    state = ref.dev_state()
    p = dev_bf16(n)
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    slots = [dev_bf16(slot_elems(lay_o, W)) for _ in range(6)]
    ups = [torch.cuda.Stream() for _ in range(n_up)]
    sts = [torch.cuda.Stream(), torch.cuda.Stream()]
    eng = zs.zs_stream_create(lay, 3, slots, ups[0] if n_up == 1 else ups,
                              sts)
    wide = torch.empty(state.numel() + 4, dtype=torch.float32,
                       device="cuda")
    with pytest.raises(zs.ZsError) as e:             # misaligned state
        zs.zs_stream_step_begin(eng, wide[1:], p, flat, step=1, **HP)
    assert e.value.code == -2
    with pytest.raises(ValueError):                  # state too short
        zs.zs_stream_step_begin(eng, state[:-4], p, flat, step=1, **HP)
    order = list(range(nb))[::-1]
    random.Random(3).shuffle(order)
    for t in (1, 2):
        ref.oracle_step(t)
        src = bucket_pool(ref, full, t, host=arrival != "device")
        torch.cuda.synchronize()        # inputs ready before the engine
        zs.zs_stream_step_begin(eng, state, p, flat, step=t, **HP)
        for b_id in order:
            zs.zs_stream_arrive(eng, b_id, src[b_id])
        if t == 2:
            with pytest.raises(zs.ZsError) as e:
                zs.zs_stream_arrive(eng, order[0], src[order[0]])
            assert e.value.code == -1
        assert zs.zs_stream_step_end(eng) == nb
        ref.check(state, f"engine {arrival} t={t}", p=p, flat=flat,
                  flat_before=flat0)
    zs.zs_stream_free(eng)


@pytest.mark.parametrize("seed", range(12))
def test_stream_engine_random_configs(seed):
    """The streaming engine under seeded random configurations: W from 2 to
    64 (compiled and runtime), group 1..16,
    a ring from the minimum (n_slots = group) to group + 5 slots, 1..3 step
    streams, 1..4 upload streams, random layouts, ranks and arrival orders,
    three steps (slots and launch events reused across steps); state and
    flat output equal the oracle's after every step, bit for bit."""
    rng = random.Random(900 + seed)
    W = rng.choice([2, 3, 4, 8, 12, 16, 64])
    numels = [rng.choice([7, 129, 1000, 4096, 9000, 33333, 70000])
              for _ in range(rng.randint(3, 12))]
    cap = W * 256 * rng.choice([1, 2, 5, 13])
    rank = rng.randrange(W)
    ref, flat, flat0 = engine_case(numels, W, rank, cap=cap,
                                   warm=(1e-4, 1e-8), seed=seed)
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    nb = len(lay_o.buckets)
    group = rng.randint(1, min(16, nb))
    n_slots = group + rng.choice([0, 0, 1, group, 5])
    n_streams = rng.randint(1, 3)
    n_up = rng.choice([1, 1, 2, 3, 4])
    say(f"case engine seed={seed} W={W} buckets={nb} group={group} "
        f"slots={n_slots} streams={n_streams} upload streams={n_up}")
    state = ref.dev_state()
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    slots = [dev_bf16(slot_elems(lay_o, W)) for _ in range(n_slots)]
    ups = [torch.cuda.Stream() for _ in range(n_up)]
    sts = [torch.cuda.Stream() for _ in range(n_streams)]
    eng = zs.zs_stream_create(lay, group, slots,
                              ups[0] if n_up == 1 else ups, sts)
    for t in (1, 2, 3):
        ref.oracle_step(t)
        pool = bucket_pool(ref, full, t)
        torch.cuda.synchronize()
        order = list(range(nb))
        rng.shuffle(order)
        zs.zs_stream_step_begin(eng, state, None, flat, step=t, **HP)
        for b_id in order:
            zs.zs_stream_arrive(eng, b_id, pool[b_id])
        assert zs.zs_stream_step_end(eng) == nb
        ref.check(state, f"engine seed={seed} t={t}", flat=flat,
                  flat_before=flat0)
    zs.zs_stream_free(eng)


def test_stream_engine_steps_back_to_back():
    """Steps queued with no host synchronisation between them: a ring of
    twice the bucket count (so no slot of a later step was read before and
    no slot-reuse wait orders anything), one bucket per launch over two
    step streams with an odd bucket count (so every bucket's launch changes
    stream from one step to the next), two upload streams; three steps,
    then the state, the shard and the flat buffer against the oracle, bit
    for bit."""
    W, rank = 4, 2
    numels = [7 * 4 * 256 * 600]         # 7 buckets of 600 x 256 elements
    cap = W * 256 * 600 * 2
    ref, flat, flat0 = engine_case(numels, W, rank, cap=cap,
                                   warm=(1e-4, 1e-8), seed=5)
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    nb = len(lay_o.buckets)
    assert nb == 7
    say(f"case engine back to back W={W} buckets={nb}")
    state = ref.dev_state()
    p = dev_bf16(n)
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    pools = {}
    for t in (1, 2, 3):
        ref.oracle_step(t)
        pools[t] = bucket_pool(ref, full, t)
    slots = [dev_bf16(slot_elems(lay_o, W)) for _ in range(2 * nb)]
    ups = [torch.cuda.Stream(), torch.cuda.Stream()]
    sts = [torch.cuda.Stream(), torch.cuda.Stream()]
    eng = zs.zs_stream_create(lay, 1, slots, ups, sts)
    torch.cuda.synchronize()              # inputs ready; none after this
    for t in (1, 2, 3):
        zs.zs_stream_step_begin(eng, state, p, flat, step=t, **HP)
        for b_id in range(nb):
            zs.zs_stream_arrive(eng, b_id, pools[t][b_id])
        assert zs.zs_stream_step_end(eng) == nb
    ref.check(state, "engine back to back", p=p, flat=flat,
              flat_before=flat0)
    zs.zs_stream_free(eng)


def test_stream_engine_70b_buckets_minimal_ring_host_arrival():
    """The Llama-3-70B-shaped workload's bucket shape at W = 16 (25 MiB
    buckets, 819,200-element slices): 40 full buckets arriving from pinned
    host memory, in reverse order, through the smallest ring (4 slots,
    groups of 4, two step streams), so every slot is overwritten as soon as
    the launch that read it is done; after each of two steps the whole state
    and the flat buffer equal the oracle's, bit for bit."""
    W, rank = 16, 3
    numels = [40 * 16 * 819200]
    ref, flat, flat0 = engine_case(numels, W, rank, sigma=1e-4)
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    nb = len(lay_o.buckets)
    assert nb == 40 and lay_o.buckets[0].slice_numel == 819200
    say(f"case engine 70b buckets W={W} buckets={nb} pinned host")
    state = ref.dev_state()
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    slots = [dev_bf16(slot_elems(lay_o, W)) for _ in range(4)]
    up = torch.cuda.Stream()
    sts = [torch.cuda.Stream(), torch.cuda.Stream()]
    eng = zs.zs_stream_create(lay, 4, slots, up, sts)
    for t in (1, 2):
        ref.oracle_step(t)
        src = bucket_pool(ref, full, t, host=True)
        torch.cuda.synchronize()
        zs.zs_stream_step_begin(eng, state, None, flat, step=t, **HP)
        for b_id in reversed(range(nb)):
            zs.zs_stream_arrive(eng, b_id, src[b_id])
        assert zs.zs_stream_step_end(eng) == nb
        ref.check(state, f"engine 70b buckets t={t}", flat=flat,
                  flat_before=flat0)
        del src
    zs.zs_stream_free(eng)


@pytest.mark.parametrize("tensors", [False, True])
def test_prefetch_pipeline_matches_the_oracle(tensors):
    """The ZeRO-3 prefetch object (zs_prefetch_*) driven as an FSDP forward:
    each unit (here every tensor, plus two multi-tensor spans) is issued
    one unit ahead into a ring of two buffers; a compute stream acquires
    it, copies it out and releases it; every copy equals the oracle's
    gather.  Out-of-order calls are refused."""
    W = 4
    numels = TENSOR_LIST + [5000, 7, 129, 70000]
    if tensors:
        lays = [build_tensor_layout(numels, W, r) for r in range(W)]
        lay = zs.zs_layout_build_tensors(numels, W, 0)
    else:
        cap = W * 256 * 37
        lays = [build_layout(numels, W, r, cap) for r in range(W)]
        lay = zs.zs_layout_build(numels, W, 0, cap)
    lay_o = lays[0]
    F = lay_o.flat_numel
    say(f"case prefetch W={W} tensors={tensors}")
    shards_h = [synth.cpu_bits16(l.shard_numel, 6, synth.TAG_SENTINEL, 0, r,
                                 0) for r, l in enumerate(lays)]
    shards = [torch.from_numpy(x.view(np.int16)).cuda() for x in shards_h]
    if tensors:
        full = gather_tensors(numels, W, shards_h, 0, F)
    else:
        full = np.zeros(F, np.uint16)
        for l, sh in zip(lays, shards_h):
            pack_flat(l, sh, full)
    offs = lay_o.tensor_flat_off
    units = [(o, o + k) for o, k in zip(offs, numels)]
    units += [(offs[1], offs[5] + numels[5]), (offs[0], F)]
    units = [(lo // 8 * 8, hi) for lo, hi in units]
    biggest = max(hi - lo for lo, hi in units)
    bufs = [dev_bf16(biggest) for _ in range(2)]
    gs, cs = torch.cuda.Stream(), torch.cuda.Stream()
    pf = zs.zs_prefetch_create(lay, shards, bufs, gs)
    outs = [dev_bf16(hi - lo) for lo, hi in units]
    torch.cuda.synchronize()
    slots = [zs.zs_prefetch_issue(pf, *units[0])]
    for u, (lo, hi) in enumerate(units):
        if u + 1 < len(units):
            slots.append(zs.zs_prefetch_issue(pf, *units[u + 1]))
        buf = zs.zs_prefetch_acquire(pf, slots[u], cs)
        with torch.cuda.stream(cs):
            outs[u].copy_(buf[:hi - lo])
        zs.zs_prefetch_release(pf, slots[u], cs)
    torch.cuda.synchronize()
    for (lo, hi), o in zip(units, outs):
        assert np.array_equal(np16(o), full[lo:hi]), (lo, hi)
    # out of order: two buffers, both issued, a third issue must wait
    a = zs.zs_prefetch_issue(pf, *units[0])
    b_ = zs.zs_prefetch_issue(pf, *units[1])
    with pytest.raises(zs.ZsError) as e:
        zs.zs_prefetch_issue(pf, *units[2])
    assert e.value.code == -1
    with pytest.raises(zs.ZsError) as e:
        zs.zs_prefetch_release(pf, a, cs)            # not acquired
    assert e.value.code == -1
    for sl in (a, b_):
        zs.zs_prefetch_acquire(pf, sl, cs)
        zs.zs_prefetch_release(pf, sl, cs)
    with pytest.raises(zs.ZsError) as e:
        zs.zs_prefetch_issue(pf, 0, biggest + 8)     # above the buffers
    assert e.value.code == -3
    # ranges outside the flat buffer, including ones whose length does not
    # fit in 64 bits, are refused before anything is queued
    for lo, hi in ((-8, 8), (16, 8), (F // 8 * 8, F + 8),
                   (-(1 << 62), 1 << 62)):
        with pytest.raises(zs.ZsError) as e:
            zs.zs_prefetch_issue(pf, lo, hi)
        assert e.value.code == -3, (lo, hi)
    lo, hi = units[0]
    sl = zs.zs_prefetch_issue(pf, lo, hi)            # still usable
    buf = zs.zs_prefetch_acquire(pf, sl, cs)
    with torch.cuda.stream(cs):
        outs[0].copy_(buf[:hi - lo])
    zs.zs_prefetch_release(pf, sl, cs)
    torch.cuda.synchronize()
    assert np.array_equal(np16(outs[0]), full[lo:hi])
    zs.zs_prefetch_free(pf)


TENSOR_LIST = [1000, 70000, 7, 129, 20000, 9000, 3, 65536, 300000, 512]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W", [1, 3, 8])
def test_whole_tensor_step(W, layout):
    """Whole-tensor shard assignment: every rank's step over its own
    tensors, bf16 result into the flat buffer at the tensors' offsets;
    against the oracle on the oracle's whole-tensor layout, bit for bit;
    other positions of the flat buffer untouched."""
    for rank in sorted({0, W - 1}):
        say(f"case whole-tensor W={W} rank={rank} {layout}")
        c = Case(TENSOR_LIST, W, rank, layout=layout, tensors=True,
                 warm=(1e-4, 1e-8), seed=W, stride_pad=8)
        F = c.lay_o.flat_numel
        flat = dev_bf16(F)
        synth.dev_bits16(flat, 3, synth.TAG_SENTINEL, 0, rank, 0)
        want = synth.cpu_bits16(F, 3, synth.TAG_SENTINEL, 0, rank, 0)
        for t in (1, 2, 3):
            c.step(t, full_flat=flat)
        torch.cuda.synchronize()
        pack_flat(c.lay_o, c.op, want)
        assert np.array_equal(np16(flat), want)


# 75 tensors of ragged sizes (tile-boundary sizes among them): at W = 1 one
# rank owns all 75, at W = 2 about 37 and at W = 3 about 25, against 32
# members per launch (three, two and one launches of the whole-shard step)
_many = random.Random(11)
MANY_TENSORS = [_many.choice([1, 7, 129, 4000, 8191, 8192, 8193, 16385,
                              20000]) + k % 5 for k in range(75)]


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("W", [1, 2, 3])
def test_whole_tensor_step_many_tensors(W, layout):
    """Whole-tensor assignment with more owned tensors than one launch takes:
    the step, the state conversions and the flat output split over several
    launches, bit for bit against the oracle; positions of other ranks'
    tensors in the flat buffer untouched; zs_state_unpack returns the
    oracle's master, m and v."""
    rank = W - 1
    say(f"case whole-tensor many W={W} rank={rank} {layout}")
    c = Case(MANY_TENSORS, W, rank, layout=layout, tensors=True,
             warm=(1e-4, 1e-8), seed=3 + W, stride_pad=8)
    assert len(c.lay_o.buckets) > (32 if W < 3 else 16)
    F = c.lay_o.flat_numel
    flat = dev_bf16(F)
    synth.dev_bits16(flat, 5, synth.TAG_SENTINEL, 0, rank, 0)
    want = synth.cpu_bits16(F, 5, synth.TAG_SENTINEL, 0, rank, 0)
    for t in (1, 2):
        c.step(t, full_flat=flat)
    torch.cuda.synchronize()
    pack_flat(c.lay_o, c.op, want)
    assert np.array_equal(np16(flat), want)
    n = c.n
    outs = [dev_f32(n) for _ in range(3)]
    for o in outs:
        o.fill_(float("nan"))
    zs.zs_state_unpack(c.lay, c.state, *outs)
    torch.cuda.synchronize()
    for got, ref in zip(outs, (c.om, c.omm, c.ov)):
        assert np.array_equal(npf(got).view(np.uint32), ref.view(np.uint32))


def test_whole_tensor_pure_bf16_and_pack():
    W = 3
    for rank in range(W):
        lay_o = build_tensor_layout(TENSOR_LIST, W, rank)
        lay = zs.zs_layout_build_tensors(TENSOR_LIST, W, rank)
        n, F = lay_o.shard_numel, lay_o.flat_numel
        say(f"case whole-tensor bf16 rank={rank} shard={n}")
        pad = S.padding_runs(n, lay_o.chunks)
        om, omm, ov = S.cpu_state(0, n, 0.02, 1, pad, (1e-4, 1e-8))
        p16 = O.bf16_round(om)
        state = dev_f32(n_tiles(lay_o) * 2 * TILE)
        zs.zs_state_mv_pack(lay, torch.from_numpy(omm.copy()).cuda(),
                            torch.from_numpy(ov.copy()).cuda(), state)
        host_flat = synth.cpu_bits16(F, 8, synth.TAG_SENTINEL, 0, 0, 0)
        pack_flat(lay_o, p16, host_flat)
        flat = torch.from_numpy(host_flat.view(np.int16)).cuda()
        G = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
        for t in (1, 2):
            S.dev_grads(G, W, n, t, 1e-3, 1, pad)
            zs.zs_step_bf16(lay, G, state, flat, params_flat=True,
                            grad_stride=n, step=t, **HP)
            O.step_bf16(S.cpu_grads(W, 0, n, t, 1e-3, 1, pad), p16, omm, ov,
                        OHP, t)
        torch.cuda.synchronize()
        want = synth.cpu_bits16(F, 8, synth.TAG_SENTINEL, 0, 0, 0)
        pack_flat(lay_o, p16, want)
        assert np.array_equal(np16(flat), want)
        m_g, v_g = from_tiled_rows(lay_o, npf(state), 2)
        assert np.array_equal(m_g, omm) and np.array_equal(v_g, ov)
        # zs_pack: flat positions and per-tensor storage
        shard = torch.from_numpy(p16.view(np.int16).copy()).cuda()
        out = dev_bf16(F)
        out.view(torch.int16).fill_(0x5a5a)
        tensors = [dev_bf16(k) for k in TENSOR_LIST]
        for x in tensors:
            x.view(torch.int16).fill_(0x1111)
        ptrs = torch.tensor([x.data_ptr() for x in tensors],
                            dtype=torch.int64, device="cuda")
        chunks = zs.zs_layout_chunks(lay)
        raw = np.frombuffer(zs.chunks_bytes(chunks), np.uint8).copy()
        zs.zs_pack(lay, shard, out, torch.from_numpy(raw).cuda(),
                   len(chunks), ptrs)
        torch.cuda.synchronize()
        want = np.full(F, 0x5a5a, np.uint16)
        pack_flat(lay_o, p16, want)
        assert np.array_equal(np16(out), want)
        ref_t = [np.full(k, 0x1111, np.uint16) for k in TENSOR_LIST]
        pack_tensors(lay_o, p16, ref_t)
        for x, r_ in zip(tensors, ref_t):
            assert np.array_equal(np16(x), r_)


@pytest.mark.parametrize("W", [3, 8])
def test_whole_tensor_ranks_reassemble_to_the_unsharded_step(W):
    """The all-reduce equivalence with whole tensors: every rank steps its
    own tensors into one shared flat buffer; it equals the oracle's step on
    the whole mean gradient, bit for bit."""
    lay0 = build_tensor_layout(TENSOR_LIST, W, 0)
    F = lay0.flat_numel
    pad = np.ones(F, bool)
    for s0, k in zip(lay0.tensor_flat_off, TENSOR_LIST):
        pad[s0:s0 + k] = False
    fullG = [np.zeros((W, F), np.uint16) for _ in range(2)]
    for t in (1, 2):
        for s_ in range(W):
            fullG[t - 1][s_] = synth.cpu_normal_bf16(F, 0, synth.TAG_GRAD, t,
                                                     s_, 0, 1e-3)
        fullG[t - 1][:, pad] = 0
    full_master = synth.cpu_normal_f32(F, 0, synth.TAG_MASTER, 0, 0, 0, 0.02)
    full_master[pad] = 0
    flat = dev_bf16(F)
    flat.view(torch.int16).fill_(0x7fc0)
    for r in range(W):
        say(f"case whole-tensor all-ranks W={W} rank={r}")
        lay_o = build_tensor_layout(TENSOR_LIST, W, r)
        lay = zs.zs_layout_build_tensors(TENSOR_LIST, W, r)
        if lay_o.shard_numel == 0:
            continue
        idx = np.concatenate([np.arange(b.flat_off, b.flat_off + b.numel)
                              for b in lay_o.buckets])
        n = idx.size
        master = torch.from_numpy(full_master[idx].copy()).cuda()
        state = dev_f32(n_tiles(lay_o) * 3 * TILE)
        zs.zs_state_pack(lay, master, None, None, state)
        for t in (1, 2):
            G = torch.from_numpy(np.ascontiguousarray(
                fullG[t - 1][:, idx]).view(np.int16)).cuda()
            zs.zs_step(lay, G, state, None, flat, grad_stride=n, step=t,
                       **HP)
        torch.cuda.synchronize()
    om = full_master.copy()
    omm = np.zeros(F, np.float32)
    ov = np.zeros(F, np.float32)
    for t in (1, 2):
        acc = O.bf16_to_f32(fullG[t - 1][0]).copy()
        for s_ in range(1, W):
            acc = acc + O.bf16_to_f32(fullG[t - 1][s_])
        p16 = O.adamw(acc / np.float32(W), om, omm, ov, OHP, t)
    assert np.array_equal(np16(flat), p16)


def test_whole_tensor_bucket_groups_and_gather():
    """Per-tensor bucket steps in groups of two (shuffled) match the
    oracle's step of the whole shard after each of two steps, bit for bit;
    zs_gather of the whole-tensor layout against the oracle (each tensor
    whole from its owner)."""
    W = 3
    rank = 1
    ref = Case(TENSOR_LIST, W, rank, tensors=True, gpu=False)
    lay, lay_o, n = ref.lay, ref.lay_o, ref.n
    state = ref.dev_state()
    full = torch.empty((W, n), dtype=torch.bfloat16, device="cuda")
    order = list(range(len(lay_o.buckets)))
    random.Random(4).shuffle(order)
    p_out = dev_bf16(n)
    for t in (1, 2):
        ref.oracle_step(t)
        ref.dev_grads(full, t)
        for g0 in range(0, len(order), 2):
            ids = order[g0:g0 + 2]
            stg = [dev_tiled_bucket(full, lay_o, b_id) for b_id in ids]
            zs.zs_buckets_step(lay, ids, stg, state, p_out, None,
                               grad_layout="tiled", step=t, **HP)
        ref.check(state, f"whole-tensor groups t={t}", p=p_out)
    # gather from the three ranks' shards
    lays = [build_tensor_layout(TENSOR_LIST, W, r) for r in range(W)]
    host = [synth.cpu_bits16(l_.shard_numel, 6, synth.TAG_SENTINEL, 0, r, 0)
            for r, l_ in enumerate(lays)]
    dev = [torch.from_numpy(h.view(np.int16)).cuda() if h.size else
           dev_bf16(8) for h in host]
    F = lays[0].flat_numel
    offs = lays[0].tensor_flat_off
    out = torch.empty(F + 64, dtype=torch.int16, device="cuda")
    for lo, hi in [(0, F), (offs[1], offs[5] + 9000), (offs[3], offs[3] + 7),
                   (offs[8], F - 5)]:
        out.fill_(0x5a5a)
        zs.zs_gather(lay, dev, lo, hi, out)
        got = np16(out)
        assert np.array_equal(got[:hi - lo],
                              gather_tensors(TENSOR_LIST, W, host, lo, hi))
        assert np.all(got[hi - lo:] == 0x5a5a)


@pytest.mark.parametrize("tensors", [False, True])
def test_checkpoint_resume_equals_the_uninterrupted_run(tmp_path, tensors):
    """Two steps, save, the state destroyed, restore, a third step: each
    step checked against the oracle, whose run is never interrupted, bit
    for bit; the restored state equals the saved one; another rank's layout
    is refused and its state left as it was."""
    W, rank = 3, 1
    say(f"case checkpoint W={W} rank={rank} tensors={tensors}")
    c = Case(TENSOR_LIST, W, rank, layout="tiled", tensors=tensors,
             warm=(1e-4, 1e-8), seed=7)
    c.step(1)
    c.step(2)
    torch.cuda.synchronize()
    snap = c.state.clone()
    path = tmp_path / "rank1.zsck"
    zs.zs_checkpoint_save(c.lay, path, c.state, step=2)
    assert path.exists() and not (tmp_path / "rank1.zsck.tmp").exists()
    c.state.fill_(float("nan"))
    build = zs.zs_layout_build_tensors if tensors else zs.zs_layout_build
    other = build(TENSOR_LIST, W, 2)
    other_state = dev_f32(zs.zs_layout_tiles(other) * 3 * TILE)
    other_state.fill_(-7.0)
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_checkpoint_load(other, path, other_state)
    assert ei.value.code == zs.ZS_EMISMATCH
    assert bool((other_state == -7.0).all())
    assert zs.zs_checkpoint_load(c.lay, path, c.state) == 2
    torch.cuda.synchronize()
    assert torch.equal(c.state.view(torch.int32), snap.view(torch.int32))
    c.step(3)


def test_checkpoint_pure_bf16_large_and_damaged(tmp_path):
    """The two-row state of the pure-bf16 step at GPT-2 size (187 MB with
    three rows, over three staging pieces): round trips bit for bit;
    a row-count mismatch is refused; a later save replaces an earlier one;
    a flipped payload byte or a truncated file fails the load."""
    w = wl.presets()["gpt2"]
    lay_o = build_layout(w.numels, w.world, 0)
    lay = zs.zs_layout_build(w.numels, w.world, 0)
    say(f"case checkpoint gpt2 tiles={n_tiles(lay_o)}")
    s3 = dev_state(lay, lay_o, 0.02, warm=(1e-4, 1e-8))
    assert s3.numel() * 4 > 2 * (64 << 20)
    back = torch.empty_like(s3)
    back.fill_(float("nan"))
    path = tmp_path / "gpt2.zsck"
    zs.zs_checkpoint_save(lay, path, s3, step=11)
    assert zs.zs_checkpoint_load(lay, path, back) == 11
    assert torch.equal(back.view(torch.int32), s3.view(torch.int32))
    # two rows: m and v of the pure-bf16 state
    s2 = s3[:n_tiles(lay_o) * 2 * TILE]
    zs.zs_checkpoint_save(lay, path, s2, step=12, rows=2)
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_checkpoint_load(lay, path, back)
    assert ei.value.code == zs.ZS_EMISMATCH
    b2 = back[:n_tiles(lay_o) * 2 * TILE]
    b2.fill_(0.0)
    assert zs.zs_checkpoint_load(lay, path, b2, rows=2) == 12
    assert torch.equal(b2.view(torch.int32), s2.view(torch.int32))
    raw = bytearray(path.read_bytes())
    assert len(raw) == 64 + s2.numel() * 4 + 8
    raw[64 + 5 * (64 << 20) // 4] ^= 0x10
    path.write_bytes(bytes(raw))
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_checkpoint_load(lay, path, b2, rows=2)
    assert ei.value.code == zs.ZS_EIO
    path.write_bytes(bytes(raw[:-100]))
    with pytest.raises(zs.ZsError) as ei:
        zs.zs_checkpoint_load(lay, path, b2, rows=2)
    assert ei.value.code == zs.ZS_EIO


def test_two_runs_are_bit_identical():
    w = wl.presets()["tiny"]
    outs = []
    for _ in range(2):
        c = Case(w.numels, w.world, 1, layout="tiled")
        for t in (1, 2, 3):
            c.step(t, check=False)
        torch.cuda.synchronize()
        outs.append(npf(c.state).view(np.uint32))
    assert np.array_equal(outs[0], outs[1])


def test_step_and_pack_replay_in_a_graph():
    """zs_step (tiled gradients, bf16 shard and flat output), zs_pack
    (per-tensor storage through a device chunk table) and zs_pack_noalloc
    (flat output alone) captured in one HIP graph on torch's capture stream
    and replayed three times, with the process's own eager work and a
    synchronisation between replays: after every replay the graph's buffers
    equal those of the same calls run eagerly on a twin set, bit for bit,
    and both equal the oracle's steps.  None of these calls allocates or
    clears memory: they record kernel launches only."""
    numels = [1000, 70000, 129, 20000, 9000]
    c = Case(numels, 4, 1, layout="tiled")
    lay, lay_o, n = c.lay, c.lay_o, c.n
    F = lay_o.flat_numel
    say(f"case graph replay W=4 rank=1 shard={n}")
    c.dev_grads(c.G, 1)
    zs.zs_grads_tile(lay, -1, c.G, c.stride, c.Gt)
    chunks = zs.zs_layout_chunks(lay)
    dch = torch.from_numpy(np.frombuffer(zs.chunks_bytes(chunks),
                                         np.uint8).copy()).cuda()
    sets = []
    for k in range(2):
        flat = dev_bf16(F)
        flat.view(torch.int16).fill_(0x1234)
        flat2 = dev_bf16(F)
        flat2.view(torch.int16).fill_(0x2345)
        tens = [torch.full((m,), 7, dtype=torch.int16, device="cuda")
                for m in numels]
        ptrs = torch.tensor([t.data_ptr() for t in tens], dtype=torch.int64,
                            device="cuda")
        sets.append(dict(state=c.dev_state(), p=dev_bf16(n), flat=flat,
                         flat2=flat2, tens=tens, ptrs=ptrs))
    flat_before = np16(sets[0]["flat"])
    flat2_before = np16(sets[0]["flat2"])

    def calls(k):
        d = sets[k]
        zs.zs_step(lay, c.Gt, d["state"], d["p"], d["flat"],
                   grad_layout="tiled", step=1, **HP)
        zs.zs_pack(lay, d["p"], None, dch, len(chunks), d["ptrs"])
        zs.zs_pack_noalloc(lay, d["p"], d["flat2"], None)

    def snapshot(k):
        d = sets[k]
        return ([npf(d["state"]).view(np.uint32), np16(d["p"]),
                 np16(d["flat"]), np16(d["flat2"])] +
                [t.cpu().numpy() for t in d["tens"]])

    # both sets once, eagerly (the kernels are loaded before the capture)
    calls(0)
    calls(1)
    c.oracle_step(1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(0)
    torch.cuda.synchronize()
    junk = torch.ones(1 << 20, device="cuda")
    for r in range(3):
        g.replay()
        junk.mul_(1.5).add_(1.0)            # the process's own eager work
        calls(1)
        c.oracle_step(1)
        torch.cuda.synchronize()
        a, b = snapshot(0), snapshot(1)
        for i, (x, y) in enumerate(zip(a, b)):
            assert np.array_equal(x, y), f"replay {r}: buffer {i}"
        c.check(sets[1]["state"], f"graph replay {r}", p=sets[1]["p"],
                flat=sets[1]["flat"], flat_before=flat_before)
        ref2 = flat2_before.copy()
        pack_flat(lay_o, c.op, ref2)
        assert np.array_equal(np16(sets[0]["flat2"]), ref2), \
            f"replay {r}: no-alloc flat pack"
        ts = [np.full(m, 7, np.uint16) for m in numels]
        pack_tensors(lay_o, c.op, ts)
        for k, (t, want) in enumerate(zip(sets[0]["tens"], ts)):
            assert np.array_equal(t.cpu().numpy().view(np.uint16), want), \
                f"replay {r}: tensor {k}"


def test_grads_tile_across_launches():
    """zs_grads_tile over a slice of more tiles than one launch covers (a
    single 35 M-element bucket at W = 2: 4273 tiles, launches of 4096): the
    tiles on both sides of the split, the ragged last tile and its zero
    padding equal the tiling rule, for the whole-shard call and the
    one-bucket call, bit for bit."""
    W, numels = 2, [40_000_000, 30_000_000]
    lay_o = build_layout(numels, W, 1, 0)
    lay = zs.zs_layout_build(numels, W, 1, 0)
    n = lay_o.shard_numel
    nt = n_tiles(lay_o)
    assert len(lay_o.buckets) == 1 and nt > 4096 + 1
    say(f"case grads tile across launches W={W} shard={n} tiles={nt}")
    stride = n + 24
    host = np.stack([synth.cpu_bits16(stride, 9, synth.TAG_SENTINEL, 0, s, 0)
                     for s in range(W)])
    dG = torch.from_numpy(host.view(np.int16)).cuda()
    pick = [0, 1, 4095, 4096, 4097, nt - 2, nt - 1]
    for bucket in (-1, 0):
        tiled = torch.empty(nt * W * TILE, dtype=torch.int16, device="cuda")
        tiled.fill_(0x5a5a)
        zs.zs_grads_tile(lay, bucket, dG, stride, tiled)
        got = np16(tiled).reshape(nt, W, TILE)
        for t in pick:
            a = t * TILE
            k = min(TILE, n - a)
            for s in range(W):
                want = np.zeros(TILE, np.uint16)
                want[:k] = host[s, a:a + k]
                assert np.array_equal(got[t, s], want), (bucket, t, s)


def test_state_pack_across_launches():
    """zs_state_pack over a slice of more tiles than one launch covers (a
    single 35 M-element bucket at W = 2: 4273 tiles, launches of 4096), with
    all three rows read (one-wave workgroups) and with the master alone (m
    and v written as zeros, 256-thread workgroups): the tiles on both sides
    of the split and the ragged last tile equal the tiling rule, bit for
    bit; the unpack returns the arrays."""
    W, numels = 2, [40_000_000, 30_000_000]
    lay_o = build_layout(numels, W, 1, 0)
    lay = zs.zs_layout_build(numels, W, 1, 0)
    n = lay_o.shard_numel
    nt = n_tiles(lay_o)
    assert len(lay_o.buckets) == 1 and nt > 4096 + 1
    say(f"case state pack across launches W={W} shard={n} tiles={nt}")
    arrs = [synth.cpu_normal_f32(n, 11, tag, 0, 0, 0, 1.0)
            for tag in (synth.TAG_MASTER, synth.TAG_M, synth.TAG_V)]
    dev = [torch.from_numpy(a).cuda() for a in arrs]
    pick = [0, 1, 4095, 4096, 4097, nt - 2, nt - 1]
    for rows in ("all", "master"):
        state = dev_f32(nt * 3 * TILE)
        state.fill_(float("nan"))
        if rows == "all":
            zs.zs_state_pack(lay, *dev, state)
        else:
            zs.zs_state_pack(lay, dev[0], None, None, state)
        got = npf(state).view(np.uint32).reshape(nt, 3, TILE)
        for t in pick:
            a = t * TILE
            k = min(TILE, n - a)
            for r in range(3):
                want = np.zeros(TILE, np.float32)
                if rows == "all" or r == 0:
                    want[:k] = arrs[r][a:a + k]
                assert np.array_equal(got[t, r], want.view(np.uint32)), \
                    (rows, t, r)
        if rows == "all":
            outs = [dev_f32(n) for _ in range(3)]
            zs.zs_state_unpack(lay, state, *outs)
            for o, x in zip(outs, arrs):
                assert np.array_equal(npf(o).view(np.uint32),
                                      x.view(np.uint32))


def test_step_is_deterministic_run_to_run():
    """Two runs of the same step on the same inputs, one after the other on
    separate copies of the state and outputs, give the same bits (GPT-2-
    shaped W = 8 shard, tiled gradients, three steps)."""
    w = wl.presets()["gpt2"]
    c = Case(w.numels, w.world, 3, layout="tiled")
    lay, n = c.lay, c.n
    F = c.lay_o.flat_numel
    say(f"case determinism gpt2 W={w.world} rank=3 shard={n}")
    runs = []
    for _ in range(2):
        st = c.dev_state()
        p = dev_bf16(n)
        flat = dev_bf16(F)
        flat.view(torch.int16).fill_(0)
        for t in (1, 2, 3):
            c.dev_grads(c.G, t)
            zs.zs_grads_tile(lay, -1, c.G, c.stride, c.Gt)
            zs.zs_step(lay, c.Gt, st, p, flat, grad_layout="tiled", step=t,
                       **HP)
        torch.cuda.synchronize()
        runs.append((npf(st).view(np.uint32), np16(p), np16(flat)))
    for x, y in zip(*runs):
        assert np.array_equal(x, y)
