"""The step's edge values on the GPU, bit for bit against the oracle.

The oracle's own pins (tests/test_oracle_step.py) fix its results on signed
zeros, bf16 subnormals and min-normals, infinities, a gradient whose square
overflows fp32, very large masters and subnormal second moments.  Here the
same kinds of values go through every work shape of the HIP step (the
mixed-precision and the pure-bf16 form; W known at compile time and at run
time; tiled and plain gradient slices), so that the flags the bit-exactness
rests on are exercised where they act: IEEE denormals (no flush to zero),
correctly rounded divide and square root, no contraction, and the sum that
starts from the first rank's value (reduce-scatter with SUM, then the
rank-local AdamW update: CS336 lecture 8 notes, "Code example: ZeRO-1";
AdamW per the DDP-to-ZeRO blog, section 3.3).

Inputs are one seeded period of P elements (P prime, so the pattern drifts
across tiles, workgroups and lanes) repeated over a one-bucket shard of up
to 4100 tiles; the oracle steps the period once, and every element of the
GPU result is compared with it.  The state and the tiled gradients are
placed by plain tensor indexing (a one-bucket shard's element j sits in
tile j // 8192 at position j % 8192), not by the library's conversions.
NaN positions must agree; NaN bits may differ (the CPU's and the GPU's
default NaN differ in sign), every other value must be identical.
"""

import numpy as np
import pytest
import torch

import zero_sharded_optimizer_shard_amd as zs
from oracle import step as O
from oracle.layout import build_layout
from tiles import n_tiles as count_tiles

pytestmark = pytest.mark.gpu

T = 8192                     # elements per tile of the tiled layouts
PERIOD = 49157               # prime

HPS = {
    "default": dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8,
                    weight_decay=0.1),
    # eps a subnormal and no decay: the denominator is the scaled root
    # alone for most elements, so the divide sees subnormal operands
    "eps subnormal": dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-45,
                          weight_decay=0.0),
}

# bf16 bit patterns of the gradients
POS0, NEG0 = 0x0000, 0x8000
SUB, NSUB, SUBMAX = 0x0001, 0x8001, 0x007F          # subnormals
MINN, NMINN = 0x0080, 0x8080                        # smallest normals
INF, NINF, QNAN = 0x7F80, 0xFF80, 0x7FC0
SQ_OVF, NSQ_OVF = 0x7F00, 0xFF00                    # 2^127: g*g overflows
BIG18, NBIG18 = 0x5D5E, 0xDD5E                      # about 1e18
MAXF = 0x7F7F                                       # largest finite
ONE, HALF_ULP = 0x3F80, 0x3380                      # 1.0 and 2^-24
FINITE_EDGES = np.array([POS0, NEG0, SUB, NSUB, SUBMAX, MINN, NMINN, SQ_OVF,
                         NSQ_OVF, BIG18, NBIG18, MAXF, ONE, HALF_ULP,
                         0x0100, 0x8100, 0x3A83, 0xBA83], np.uint16)
ALL_EDGES = np.concatenate([FINITE_EDGES,
                            np.array([INF, NINF, QNAN], np.uint16)])
# finite edges whose sums stay finite at any W here
SMALL_EDGES = np.array([e for e in FINITE_EDGES
                        if e not in (SQ_OVF, NSQ_OVF, MAXF)], np.uint16)
# how often each column kind of edge_gradients is drawn: the kinds that
# make the state Inf or NaN for good (5, 8, 9, 10, 11) stay rare, so that
# the second step still sees mostly finite state
KIND_WEIGHTS = np.array([8, 6, 8, 10, 8, 2, 10, 10, 2, 2, 2, 2, 10, 10, 10],
                        np.float64)
KIND_WEIGHTS /= KIND_WEIGHTS.sum()

F32 = np.float32
MASTERS = np.array([0.0, -0.0, 1e-30, -3.0, 3e38, -3e38, 1e-40, -1e-44,
                    1.0, 1.17549435e-38, 3.4028235e38, 0.02, -0.02],
                   np.float32)
MOMENTS1 = np.array([0.0, -0.0, 1e-42, -1e-40, 1e-3, -3e30, 3e38, 1e-30,
                     -1e-38], np.float32)
MOMENTS2 = np.array([0.0, 1.4e-45, 1e-42, 1e-40, 1.17549435e-38, 1e-38,
                     1e-10, 1e30, 3e38], np.float32)


def bf16_of(x):
    """bf16 bits of float32 values that are exactly representable."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert not np.any(b & 0xFFFF)
    return (b >> 16).astype(np.uint16)


def edge_gradients(W, rng):
    """uint16 [W][PERIOD]: every element's W slices follow one of the
    column patterns below, chosen at random per element."""
    G = np.zeros((W, PERIOD), np.uint16)
    kind = rng.choice(len(KIND_WEIGHTS), PERIOD, p=KIND_WEIGHTS)
    # ordinary N(0, 1e-3) values, cut to bf16 (high halves)
    normal = (rng.normal(0, 1e-3, (W, PERIOD)).astype(np.float32)
              .view(np.uint32) >> 16).astype(np.uint16)
    for i in range(PERIOD):
        k = kind[i]
        col = G[:, i]
        if k == 0:                          # all -0: the sum stays -0
            col[:] = NEG0
        elif k == 1:
            col[:] = POS0
        elif k == 2:                        # signed zeros, mixed
            col[:] = rng.choice([POS0, NEG0], W)
        elif k == 3:                        # one subnormal kind throughout
            col[:] = rng.choice([SUB, NSUB, SUBMAX, MINN])
        elif k == 4:                        # one 2^127 among zeros: v = +Inf
            col[:] = rng.choice([POS0, NEG0], W)
            col[rng.integers(W)] = rng.choice([SQ_OVF, NSQ_OVF])
        elif k == 5:                        # anything, Inf and NaN included
            col[:] = rng.choice(ALL_EDGES, W)
        elif k == 6:                        # finite edges, finite sums
            col[:] = rng.choice(SMALL_EDGES, W)
        elif k == 7:                        # ordinary values, one subnormal
            col[:] = normal[:, i]
            col[rng.integers(W)] = rng.choice([SUB, NSUB, SUBMAX])
        elif k == 8:                        # one +-Inf among ordinary ones
            col[:] = normal[:, i]
            col[rng.integers(W)] = rng.choice([INF, NINF])
        elif k == 9:                        # +Inf and -Inf: NaN (W > 1)
            col[:] = normal[:, i]
            col[0] = INF
            col[W - 1] = NINF
        elif k == 10:                       # one NaN
            col[:] = normal[:, i]
            col[rng.integers(W)] = QNAN
        elif k == 11:                       # largest finite: the sum overflows
            col[:] = rng.choice([MAXF, SQ_OVF])
        elif k == 12:                       # x then -x: exact cancellation
            x = rng.choice(FINITE_EDGES)
            col[:] = x
            col[1::2] = x ^ 0x8000
        elif k == 13:                       # subnormals of both signs
            col[:] = rng.choice([SUB, NSUB, 0x0002, 0x8003], W)
        else:                               # about 1e18, both signs
            col[:] = rng.choice([BIG18, NBIG18, POS0], W)
    return G


def edge_state(rng):
    """fp32 master, m, v [PERIOD] from the edge sets (v >= 0), a few
    ordinary values among them, and a sprinkle of Inf/NaN masters."""
    master = rng.choice(MASTERS, PERIOD).astype(np.float32)
    ordinary = rng.random(PERIOD) < 0.2
    master[ordinary] = rng.normal(0, 0.02, ordinary.sum()).astype(np.float32)
    odd = rng.random(PERIOD) < 0.01
    master[odd] = rng.choice(np.array([np.inf, -np.inf, np.nan], F32),
                             odd.sum())
    m = rng.choice(MOMENTS1, PERIOD).astype(np.float32)
    v = rng.choice(MOMENTS2, PERIOD).astype(np.float32)
    return master, m, v


def expand(a, n):
    """Device copy of the period `a` (last axis) repeated to length n."""
    d = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    reps = -(-n // a.shape[-1])
    if d.ndim == 1:
        return d.repeat(reps)[:n].contiguous()
    return d.repeat(1, reps)[:, :n].contiguous()


def to_tiled(rows, n_tiles):
    """[R][n] device rows -> the tiled [n_tiles][R][T] layout of a
    one-bucket shard, padding zero."""
    R, n = rows.shape
    tmp = torch.zeros((R, n_tiles * T), dtype=rows.dtype, device="cuda")
    tmp[:, :n] = rows
    return tmp.view(R, n_tiles, T).permute(1, 0, 2).contiguous().view(-1)


def from_tiled(tiled, R, n_tiles, n):
    """The tiled layout back to [R][n] host rows."""
    x = tiled.view(n_tiles, R, T).permute(1, 0, 2).reshape(R, -1)[:, :n]
    return x.cpu().numpy()


def assert_periodic_equal(got, want, what):
    """Every element of got (length n) equals want[i % PERIOD] bit for bit,
    NaN positions agreeing (their bits may differ)."""
    n = got.size
    reps = n // PERIOD
    u = np.uint32 if got.dtype == np.float32 else np.uint16
    if u is np.uint32:
        isnan = np.isnan
    else:
        def isnan(b):
            return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    for part, ref in ((got[:reps * PERIOD].reshape(reps, PERIOD),
                       want[None, :]),
                      (got[reps * PERIOD:], want[:n - reps * PERIOD])):
        if part.size == 0:
            continue
        gb, rb = part.view(u), np.broadcast_to(ref, part.shape).view(u)
        gn, rn = isnan(part), np.broadcast_to(isnan(ref), part.shape)
        bad = (gn != rn) | (~gn & ~rn & (gb != rb))
        if bad.any():
            idx = np.argwhere(bad)[0]
            i = int(idx[-1])
            raise AssertionError(
                f"{what}: {int(bad.sum())} elements differ; first at period "
                f"position {i}: got {part[tuple(idx)]!r} "
                f"({int(part.view(u)[tuple(idx)]):#x}), want {ref.reshape(-1)[i]!r} "
                f"({int(ref.reshape(-1).view(u)[i]):#x})")


def one_bucket(W, tiles):
    """A one-bucket, one-tensor layout whose rank slice is `tiles` tiles,
    the last one half full; rank W - 1."""
    n_rank = tiles * T - 4096
    numels = [W * n_rank]
    lay = zs.zs_layout_build(numels, W, W - 1, 0)
    lay_o = build_layout(numels, W, W - 1, 0)
    assert count_tiles(lay_o) == tiles and len(lay_o.buckets) == 1
    assert lay_o.shard_numel == n_rank
    return lay, n_rank


# (W, tiles): which work shape runs (launches of fewer than 4096 tiles
# differ from larger ones in the workgroups allowed per CU, and at runtime W
# in the shape)
#   (2, 300)    One <64, 1, 4>, W = 2     (5, 1100)  Small, runtime W
#   (1, 4100)   One <64, 1, 4>, W = 1     (8, 4100)  One <64, 1, 8>
#   (16, 4100)  One <64, 1, 16>
#   (32, 4100)  One <64, 1, 32> tiled, Deep on plain slices
#   (64, 4100)  One <64, 1, 64> tiled, Deep on plain slices
#   (64, 300)   One <64, 1, 64> tiled, Small on plain slices
#   runtime W, 4100 tiles: one-wave workgroups with batches of 8 (5), 16
#   (12), 32 (20, 33) and 64 (100) on tiled gradients (and at W = 5 on
#   plain slices); Wave (12, 20) and Wide (33, 100) on plain slices;
#   (128, 4100): two full batches of 64; (12, 300) and (65, 300): one-wave
#   batches of 16 and of 64 + 1 below 4096 tiles on tiled gradients, Small
#   on plain slices
SHAPES = [(2, 300), (5, 1100), (1, 4100), (8, 4100), (16, 4100), (5, 4100),
          (12, 4100), (20, 4100), (32, 4100), (64, 4100), (33, 4100),
          (100, 4100), (128, 4100), (64, 300), (12, 300), (65, 300)]


@pytest.mark.parametrize("state_form", ["tiled", "plain"])
@pytest.mark.parametrize("hp_name", list(HPS))
@pytest.mark.parametrize("layout", ["tiled", "slices"])
@pytest.mark.parametrize("W,tiles", SHAPES)
def test_step_edge_values(W, tiles, layout, hp_name, state_form):
    """zs_step (tiled state) and zs_step_plain (three plain arrays)."""
    hp = HPS[hp_name]
    print(f"case edge step W={W} tiles={tiles} {layout} {hp_name} "
          f"{state_form} state", flush=True)
    rng = np.random.default_rng(1000 * W + tiles)
    lay, n = one_bucket(W, tiles)
    n_tiles = tiles
    master, m, v = edge_state(rng)
    rows = torch.stack([expand(x, n) for x in (master, m, v)])
    state = to_tiled(rows, n_tiles) if state_form == "tiled" else None

    def step(grads, t, **kw):
        if state_form == "tiled":
            zs.zs_step(lay, grads, state, p, None, step=t, **kw, **hp)
        else:
            zs.zs_step_plain(lay, grads, rows[0], rows[1], rows[2], p, None,
                             step=t, **kw, **hp)

    def read_state():
        if state_form == "tiled":
            return from_tiled(state, 3, n_tiles, n)
        return rows.cpu().numpy()

    p = torch.empty(n, dtype=torch.int16, device="cuda")
    om, omm, ov = master.copy(), m.copy(), v.copy()
    for t in (1, 2):
        Gp = edge_gradients(W, rng)
        G = expand(Gp.view(np.int16), n)
        if layout == "tiled":
            step(to_tiled(G, n_tiles), t, grad_layout="tiled")
        else:
            Gs = torch.zeros((W, n + 8), dtype=torch.int16, device="cuda")
            Gs[:, :n] = G
            step(Gs, t, grad_layout="slices", grad_stride=n + 8)
        op = O.step(Gp, om, omm, ov, O.AdamW(**hp), t)
        torch.cuda.synchronize()
        got = read_state()
        for row, name, want in ((0, "master", om), (1, "m", omm),
                                (2, "v", ov)):
            assert_periodic_equal(got[row], want, f"t={t} {name}")
        assert_periodic_equal(p.cpu().numpy().view(np.uint16), op,
                              f"t={t} bf16 param")
    # the values reached the cases they are meant for
    assert np.isinf(ov).any() and (ov[np.isfinite(ov)] > 0).any()
    assert ((ov > 0) & (ov < 1.17549435e-38)).any()      # subnormal v
    assert np.isnan(om).any()


# the pure-bf16 step's shapes: One (W = 2, 8, 16, 32, 64; Deep on plain
# slices at W >= 32; at runtime W above 8 on tiled gradients, batches of 16,
# 32 and 64 for W = 12, 33, 100), Wave (runtime W up to 8, and plain slices
# below 32), PureWide (plain slices at runtime W >= 32), Small (runtime W,
# and plain slices at W = 64, below 4096 tiles)
PURE_SHAPES = [(2, 300), (5, 1100), (64, 300), (8, 4100), (16, 4100),
               (5, 4100), (12, 4100), (32, 4100), (64, 4100), (33, 4100),
               (100, 4100)]


@pytest.mark.parametrize("layout", ["tiled", "slices"])
@pytest.mark.parametrize("W,tiles", PURE_SHAPES)
def test_pure_bf16_step_edge_values(W, tiles, layout):
    hp = HPS["default"]
    print(f"case edge bf16 step W={W} tiles={tiles} {layout}", flush=True)
    rng = np.random.default_rng(2000 * W + tiles)
    lay, n = one_bucket(W, tiles)
    master, m, v = edge_state(rng)
    p16 = O.bf16_round(master)
    # bf16 parameters at their own edges too: subnormal, largest finite
    pick = rng.random(PERIOD) < 0.1
    p16[pick] = rng.choice(np.array([0x0001, 0x8001, 0x7F7F, 0xFF7F, 0x0080],
                                    np.uint16), pick.sum())
    state = to_tiled(torch.stack([expand(x, n) for x in (m, v)]), tiles)
    params = expand(p16.view(np.int16), n)
    om, ov = m.copy(), v.copy()
    for t in (1, 2):
        Gp = edge_gradients(W, rng)
        G = expand(Gp.view(np.int16), n)
        if layout == "tiled":
            zs.zs_step_bf16(lay, to_tiled(G, tiles), state, params,
                            params_flat=False, grad_layout="tiled", step=t,
                            **hp)
        else:
            zs.zs_step_bf16(lay, G, state, params, params_flat=False,
                            grad_layout="slices", grad_stride=n, step=t,
                            **hp)
        O.step_bf16(Gp, p16, om, ov, O.AdamW(**hp), t)
        torch.cuda.synchronize()
        got = from_tiled(state, 2, tiles, n)
        assert_periodic_equal(got[0], om, f"t={t} m")
        assert_periodic_equal(got[1], ov, f"t={t} v")
        assert_periodic_equal(params.cpu().numpy().view(np.uint16), p16,
                              f"t={t} bf16 param")


# the bucket-group kernel (zs_bucket_step: a group of one bucket): One
# below 4096 tiles at compiled W (Small on plain slices at W = 64), at
# runtime W above 8 one-wave batches on tiled gradients (Small on plain
# slices), Small at runtime W up to 8; at 4096 tiles or more Wave (compiled
# and runtime W < 32), Deep at compiled W >= 32, Wide at runtime W >= 32
GROUP_SHAPES = [(2, 300), (8, 300), (16, 300), (64, 300), (5, 300),
                (12, 300), (48, 300), (8, 4100), (5, 4100), (64, 4100),
                (33, 4100)]


@pytest.mark.parametrize("layout", ["tiled", "slices"])
@pytest.mark.parametrize("W,tiles", GROUP_SHAPES)
def test_bucket_step_edge_values(W, tiles, layout):
    hp = HPS["default"]
    print(f"case edge bucket step W={W} tiles={tiles} {layout}", flush=True)
    rng = np.random.default_rng(3000 * W + tiles)
    lay, n = one_bucket(W, tiles)
    master, m, v = edge_state(rng)
    state = to_tiled(torch.stack([expand(x, n) for x in (master, m, v)]),
                     tiles)
    p = torch.empty(n, dtype=torch.int16, device="cuda")
    om, omm, ov = master.copy(), m.copy(), v.copy()
    for t in (1, 2):
        Gp = edge_gradients(W, rng)
        G = expand(Gp.view(np.int16), n)
        if layout == "tiled":
            zs.zs_bucket_step(lay, 0, to_tiled(G, tiles), state, p, None,
                              grad_layout="tiled", step=t, **hp)
        else:
            zs.zs_bucket_step(lay, 0, G, state, p, None,
                              grad_layout="slices", grad_stride=n, step=t,
                              **hp)
        op = O.step(Gp, om, omm, ov, O.AdamW(**hp), t)
        torch.cuda.synchronize()
        got = from_tiled(state, 3, tiles, n)
        for row, name, want in ((0, "master", om), (1, "m", omm),
                                (2, "v", ov)):
            assert_periodic_equal(got[row], want, f"t={t} {name}")
        assert_periodic_equal(p.cpu().numpy().view(np.uint16), op,
                              f"t={t} bf16 param")
