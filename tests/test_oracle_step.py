"""Pins of the step oracle (oracle/zs_oracle.c) against what the pages and
the mathematics fix, none of which shares code with it:

* W = 1 is plain AdamW: torch.optim.AdamW / Adam on the CPU (library).
* The first step from m = v = 0 has the closed form
  th1 = th0*(1 - lr*wd) - lr*g/(|g| + eps).
* beta1 = beta2 = 0 gives that closed form at every step.
* lr = 0 leaves the master bit-identical while the moments advance.
* A float64 evaluation of the same formula agrees to a few fp32 roundings.
* all-reduce = reduce-scatter + all-gather: every rank's shard result,
  reassembled through the layout, equals the step on the full-array mean.
* fp32 -> bf16 rounding equals torch's conversion on every high half.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import step as O
from oracle.layout import build_layout
from oracle.pack import pack_flat

F32_EPS = 2.0 ** -24          # unit roundoff of fp32


def f32(x):
    return float(np.float32(x))


def hp_f32(**kw):
    """Hyper-parameters already rounded to fp32, so torch (which works in
    double on the host side) sees exactly the values the oracle sees."""
    base = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    base.update(kw)
    return O.AdamW(**{k: f32(v) for k, v in base.items()})


def grads_bf16(W, n, step, sigma=1e-3, seed=0, base=0):
    return np.stack([synth.cpu_normal_bf16(n, seed, synth.TAG_GRAD, step, s,
                                           base, sigma) for s in range(W)])


def master_f32(n, seed=0, base=0, sigma=0.02):
    return synth.cpu_normal_f32(n, seed, synth.TAG_MASTER, 0, 0, base, sigma)


def within(x, ref, rel, abs_floor):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.all(np.abs(x - ref) <= np.maximum(rel * np.abs(ref), abs_floor))


TORCH_CASES = [
    # (grad sigma, hyper-parameters): sigma 1e-8 makes sqrt(v) comparable to
    # eps, which pins where eps sits; the large lr/wd case pins that the
    # decay multiplies the old master.
    (1.0, {}),
    (1e-3, {}),
    (1e-8, {}),
    (1.0, dict(lr=0.1, weight_decay=0.5, beta1=0.8, beta2=0.9)),
]


@pytest.mark.parametrize("sigma,kw", TORCH_CASES)
@pytest.mark.parametrize("decoupled", [True, False])
def test_w1_matches_torch_library(decoupled, sigma, kw):
    """W = 1: the step is the library's AdamW (or Adam when wd = 0).

    Bar: 1e-6 of each value plus 1e-6 of the array's largest magnitude (the
    library rounds m through a lerp and the update through addcdiv, so
    values that cancel differ by an ulp of the terms, not of the result)."""
    n = 4096
    hp = hp_f32(**kw)
    if not decoupled:
        hp = hp_f32(**{**kw, "weight_decay": 0.0})
    master = master_f32(n)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = torch.nn.Parameter(torch.from_numpy(master.copy()))
    cls = torch.optim.AdamW if decoupled else torch.optim.Adam
    opt = cls([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
              weight_decay=hp.weight_decay, foreach=False, fused=False)
    for t in range(1, 7):
        G = grads_bf16(1, n, t, sigma=sigma)
        p16 = O.step(G, master, m, v, hp, t)
        p.grad = torch.from_numpy(O.bf16_to_f32(G[0]).copy())
        opt.step()
        st = opt.state[p]
        for x, ref in ((master, p.detach().numpy()),
                       (m, st["exp_avg"].numpy()),
                       (v, st["exp_avg_sq"].numpy())):
            floor = 1e-6 * float(np.abs(ref).max())
            assert within(x, ref, 1e-6, floor)
        ref16 = p.detach().to(torch.bfloat16).view(torch.int16).numpy()
        d = np.abs(p16.astype(np.int32)
                   - ref16.view(np.uint16).astype(np.int32))
        assert d.max() <= 1


def test_first_step_closed_form():
    n, W = 8192, 4
    hp = hp_f32()
    G = grads_bf16(W, n, 1)
    th0 = master_f32(n)
    master = th0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    O.step(G, master, m, v, hp, 1)
    g = O.reduce_mean(G).astype(np.float64)
    lr, wd, eps = hp.lr, hp.weight_decay, hp.eps
    dec = th0.astype(np.float64) * (1 - lr * wd)
    upd = lr * g / (np.abs(g) + eps)
    ref = dec - upd
    bound = 4 * F32_EPS * (np.abs(dec) + np.abs(upd))
    assert np.all(np.abs(master - ref) <= bound)
    # zero gradient: no Adam update, pure decay
    z = np.zeros((W, 16), np.uint16)
    th = th0[:16].copy()
    O.step(z, th, np.zeros(16, np.float32), np.zeros(16, np.float32), hp, 1)
    assert np.array_equal(th, (th0[:16] * np.float32(1 - lr * wd)))


def test_zero_betas_closed_form_every_step():
    n, W = 4096, 3
    hp = hp_f32(beta1=0.0, beta2=0.0)
    master = master_f32(n)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 5):
        G = grads_bf16(W, n, t)
        th = master.astype(np.float64)
        O.step(G, master, m, v, hp, t)
        g = O.reduce_mean(G).astype(np.float64)
        dec = th * (1 - hp.lr * hp.weight_decay)
        upd = hp.lr * g / (np.abs(g) + hp.eps)
        bound = 4 * F32_EPS * (np.abs(dec) + np.abs(upd))
        assert np.all(np.abs(master - (dec - upd)) <= bound)
        assert np.array_equal(m, O.reduce_mean(G))


def test_zero_lr_keeps_master():
    n, W = 2048, 2
    hp = hp_f32(lr=0.0)
    th0 = master_f32(n)
    master = th0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 4):
        O.step(grads_bf16(W, n, t), master, m, v, hp, t)
    assert np.array_equal(master, th0)
    assert np.count_nonzero(m) > n // 2 and np.count_nonzero(v) > n // 2


def float64_step(G, th, m, v, hp, t):
    """The same formula evaluated in float64 from the same inputs."""
    W = G.shape[0]
    g = O.bf16_to_f32(G).astype(np.float64).sum(axis=0) / W
    b1, b2 = float(hp.beta1), float(hp.beta2)
    m = b1 * m + (1 - b1) * g
    v = b2 * v + (1 - b2) * g * g
    bc1 = 1 - b1 ** t
    bc2 = 1 - b2 ** t
    den = np.sqrt(v) / np.sqrt(bc2) + hp.eps
    th_dec = th * (1 - hp.lr * hp.weight_decay)
    upd = (hp.lr / bc1) * (m / den)
    return g, m, v, den, th_dec, upd, hp.lr / bc1


EDGE = np.array([0x0000, 0x8000, 0x0080, 0x8080, 0x0001, 0x8001, 0x3f80,
                 0xbf80, 0x5d5e, 0xdd5e, 0x2000, 0x1f80],
                np.uint16)   # +-0, min normals, denormals, +-1, +-1e18, ...


@pytest.mark.parametrize("W", [1, 2, 3, 5, 8])
def test_float64_brute_force(W):
    """Each fp32 statement may add a few roundings of its own terms; the
    bounds below allow exactly that and nothing of the size a wrong term,
    sign or index would leave."""
    n = 2048
    hp = hp_f32()
    G = grads_bf16(W, n, 1, sigma=1e-2)
    G[:, :EDGE.size] = EDGE[None, :]
    G[0, EDGE.size:2 * EDGE.size] = EDGE        # one edge value among normals
    master = master_f32(n)
    master[:4] = [0.0, -0.0, 1e-30, -3.0]
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in range(1, 5):
        th64, m64, v64 = (master.astype(np.float64), m.astype(np.float64),
                          v.astype(np.float64))
        g, m_ref, v_ref, den, th_dec, upd, ss = float64_step(G, th64, m64,
                                                            v64, hp, t)
        O.step(G, master, m, v, hp, t)
        gabs = np.abs(O.bf16_to_f32(G).astype(np.float64)).sum(axis=0) / W
        eg = (W + 1) * F32_EPS * gabs                 # error of the mean
        bm = 4 * F32_EPS * (np.abs(hp.beta1 * m64) + 0.1 * np.abs(g)) \
            + 0.1 * eg + 1e-45
        bv = 6 * F32_EPS * (np.abs(hp.beta2 * v64) + 0.05 * g * g) \
            + 0.05 * (2 * np.abs(g) + eg) * eg + 1e-45
        assert np.all(np.abs(m - m_ref) <= bm)
        assert np.all(np.abs(v - v_ref) <= bv)
        bden = 6 * F32_EPS * den + bv / np.maximum(np.sqrt(v_ref), 1e-38)
        bupd = ss * (bm / den + np.abs(m_ref) * bden / den ** 2)
        bth = 8 * F32_EPS * (np.abs(th_dec) + np.abs(upd)) + bupd + 1e-44
        assert np.all(np.abs(master - (th_dec - upd)) <= bth)
        G = grads_bf16(W, n, t + 1, sigma=1e-2)


def test_padding_stays_zero_and_nan_is_local():
    W, n = 4, 64
    hp = hp_f32()
    G = np.zeros((W, n), np.uint16)
    master = np.zeros(n, np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    G[2, 5] = 0x7fc0                              # one NaN gradient value
    for t in range(1, 4):
        p16 = O.step(G, master, m, v, hp, t)
    keep = np.ones(n, bool)
    keep[5] = False
    assert np.all(master[keep].view(np.uint32) == 0)   # +0 exactly
    assert np.all(m[keep].view(np.uint32) == 0)
    assert np.all(v[keep].view(np.uint32) == 0)
    assert np.all(p16[keep] == 0)
    assert np.isnan(master[5]) and np.isnan(m[5]) and np.isnan(v[5])


def test_gradient_square_overflow():
    """A gradient whose square overflows fp32 makes v infinite, the update
    m/inf zero, and leaves only the decay: fp32 semantics, no skip."""
    hp = hp_f32()
    G = np.full((1, 8), 0x7f00, np.uint16)          # 1.7e38
    th0 = master_f32(8)
    master = th0.copy()
    m = np.zeros(8, np.float32)
    v = np.zeros(8, np.float32)
    O.step(G, master, m, v, hp, 1)
    assert np.all(np.isinf(v)) and np.all(np.isfinite(m))
    assert np.array_equal(master, th0 * np.float32(1 - hp.lr * hp.weight_decay))


def test_reduce_mean_is_fixed_order_sum():
    W, n = 5, 1000
    G = grads_bf16(W, n, 3)
    acc = O.bf16_to_f32(G[0]).copy()
    for s in range(1, W):
        acc = acc + O.bf16_to_f32(G[s])
    assert np.array_equal(O.reduce_mean(G), acc / np.float32(W))


def test_reduce_order_is_rank_order():
    """Where fp32 rounding makes the order visible: 2^-24 is half an ulp of
    1.0, so 1 + 2^-24 + 2^-24 is 1 left to right (each addition ties to the
    even 1.0), while 2^-24 + 2^-24 + 1 is exactly 1 + 2^-23.  Slices are
    summed in rank order 0, 1, ..., W-1, starting from slice 0."""
    one, tiny = 0x3F80, 0x3380          # bf16 bits of 1.0 and 2^-24
    G = np.array([[one, tiny, tiny, one],
                  [tiny, tiny, one, tiny],
                  [tiny, one, tiny, tiny]], np.uint16)
    got = O.reduce_mean(G)
    third = np.float32(1) / np.float32(3)
    big = np.float32(1 + 2 ** -23) / np.float32(3)
    # element 0: 1, t, t -> 1; element 1: t, t, 1 -> 1 + 2^-23;
    # element 2: t, 1, t -> t + 1 = 1, + t = 1; element 3: 1, t, t -> 1
    assert got.tolist() == [third, big, third, third]
    assert third != big


def test_step_is_reduce_then_adamw():
    W, n = 3, 3000
    hp = hp_f32()
    a = [master_f32(n), np.full(n, 1e-4, np.float32),
         np.full(n, 1e-8, np.float32)]
    b = [x.copy() for x in a]
    for t in (1, 2, 7):
        G = grads_bf16(W, n, t)
        p1 = O.step(G, *a, hp, t)
        p2 = O.adamw(O.reduce_mean(G), *b, hp, t)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        assert np.array_equal(p1, p2)


@pytest.mark.parametrize("W,cap", [(2, 4096), (3, 6000), (4, 1 << 20),
                                   (5, 10240), (8, 8192)])
def test_allreduce_equals_reduce_scatter_plus_all_gather(W, cap):
    """Run the step on every rank's shard, all-gather the results through
    the layout, and compare with the step on the whole mean gradient."""
    numels = [1000, 7, 129, 4096, 300, 2047, 64]
    hp = hp_f32()
    lay0 = build_layout(numels, W, 0, cap, 256)
    F = lay0.flat_numel
    # W full local gradients over the flat buffer, zero in the padding
    pad = np.ones(F, bool)
    for s0, n in zip(lay0.tensor_flat_off, numels):
        pad[s0:s0 + n] = False
    full_master = master_f32(F)
    full_master[pad] = 0
    steps = 3
    fullG = []
    for t in range(1, steps + 1):
        Gt = grads_bf16(W, F, t)
        Gt[:, pad] = 0
        fullG.append(Gt)
    # sharded: every rank on its own slices
    out_master = np.full(F, np.nan, np.float32)
    out_m = np.full(F, np.nan, np.float32)
    out_p = np.zeros(F, np.uint16)
    for r in range(W):
        lay = build_layout(numels, W, r, cap, 256)
        idx = np.concatenate([np.arange(b.flat_off + r * b.slice_numel,
                                        b.flat_off + (r + 1) * b.slice_numel)
                              for b in lay.buckets])
        master = full_master[idx].copy()
        m = np.zeros(idx.size, np.float32)
        v = np.zeros(idx.size, np.float32)
        for t in range(1, steps + 1):
            p16 = O.step(np.ascontiguousarray(fullG[t - 1][:, idx]), master,
                         m, v, hp, t)
        pack_flat(lay, master, out_master)
        pack_flat(lay, m, out_m)
        pack_flat(lay, p16, out_p)
    # unsharded: the all-reduce mean, then the update on the whole buffer
    master = full_master.copy()
    m = np.zeros(F, np.float32)
    v = np.zeros(F, np.float32)
    for t in range(1, steps + 1):
        Gt = fullG[t - 1]
        acc = O.bf16_to_f32(Gt[0]).copy()
        for s in range(1, W):
            acc = acc + O.bf16_to_f32(Gt[s])
        p16 = O.adamw(acc / np.float32(W), master, m, v, hp, t)
    assert np.array_equal(out_master.view(np.uint32), master.view(np.uint32))
    assert np.array_equal(out_m.view(np.uint32), m.view(np.uint32))
    assert np.array_equal(out_p, p16)
    assert np.all(out_master[pad] == 0)


def test_bf16_rounding_matches_torch():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7fff, 0x8000, 0x8001, 0xffff, 0x4000,
                     0xc000], np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    got = O.bf16_round(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN with its sign
    g = got[nan]
    assert np.all((g & 0x7f80) == 0x7f80) and np.all((g & 0x7f) != 0)
    assert np.array_equal(g >> 15, (bits[nan] >> 31).astype(np.uint16))


def test_constants_first_step():
    hp = hp_f32()
    c = O.constants(hp, 1)
    b1, b2 = float(hp.beta1), float(hp.beta2)
    assert c[0] == np.float32(b1) and c[1] == np.float32(b2)
    assert c[4] == np.float32(hp.lr / (1 - b1))
    assert c[5] == np.float32(np.sqrt(1 - b2))
    assert c[6] == np.float32(1 - hp.lr * hp.weight_decay)
    # the bias corrections vanish as t grows
    c = O.constants(hp, 10_000)
    assert c[4] == np.float32(hp.lr) and c[5] == np.float32(1.0)


# ---- pure-bf16 variant (no fp32 master) ---------------------------------

def bf16_ordinal(bits):
    b = np.asarray(bits, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7fff), b)


@pytest.mark.parametrize("W", [1, 3, 8])
def test_bf16_step_is_the_mixed_step_from_the_bf16_value(W):
    """Each pure-bf16 step equals the (pinned) mixed-precision step whose
    master starts from the bf16 parameter, rounded back to bf16; the
    moments are identical.  Checked over several steps with warm moments."""
    n = 4096
    hp = hp_f32()
    p16 = O.bf16_round(master_f32(n))
    m = synth.cpu_normal_f32(n, 1, synth.TAG_M, 0, 0, 0, 1e-4)
    v = synth.cpu_normal_f32(n, 1, synth.TAG_V, 0, 0, 0, 1e-8, True)
    m2, v2 = m.copy(), v.copy()
    for t in range(1, 6):
        G = grads_bf16(W, n, t)
        master = O.bf16_to_f32(p16).copy()
        want = O.step(G, master, m2, v2, hp, t)
        O.step_bf16(G, p16, m, v, hp, t)
        assert np.array_equal(p16, want)
        assert np.array_equal(m.view(np.uint32), m2.view(np.uint32))
        assert np.array_equal(v.view(np.uint32), v2.view(np.uint32))


def test_bf16_first_step_closed_form():
    n, W = 8192, 4
    hp = hp_f32()
    G = grads_bf16(W, n, 1)
    p0 = O.bf16_round(master_f32(n))
    p = p0.copy()
    O.step_bf16(G, p, np.zeros(n, np.float32), np.zeros(n, np.float32), hp,
                1)
    g = O.reduce_mean(G).astype(np.float64)
    th0 = O.bf16_to_f32(p0).astype(np.float64)
    lr, wd, eps = hp.lr, hp.weight_decay, hp.eps
    ref = th0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    # the fp32 value is within a few roundings of ref, so its bf16 rounding
    # is ref's bf16 rounding or a neighbour
    refb = O.bf16_round(ref.astype(np.float32))
    assert np.abs(bf16_ordinal(p) - bf16_ordinal(refb)).max() <= 1


def test_bf16_zero_lr_keeps_the_parameter_and_small_updates_vanish():
    n, W = 2048, 2
    G = grads_bf16(W, n, 1)
    p0 = O.bf16_round(master_f32(n))
    p = p0.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    O.step_bf16(G, p, m, v, hp_f32(lr=0.0), 1)
    assert np.array_equal(p, p0) and np.any(m != 0)
    # parameters of 1.0: an Adam step of 1e-5 is below half an ulp of bf16
    # (2^-8 at 1.0), so with no decay the parameter never moves, step after
    # step; an fp32 master would have moved by about 3e-5 after 3 steps
    one = np.full(n, 0x3f80, np.uint16)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for t in (1, 2, 3):
        O.step_bf16(grads_bf16(W, n, t), one, m, v,
                    hp_f32(lr=1e-5, weight_decay=0.0), t)
    assert np.all(one == 0x3f80)


@pytest.mark.parametrize("threads", [1, 2, 3, 8])
def test_step_is_deterministic_over_threads_and_windows(threads):
    """The step is elementwise, so any split of a run of elements into
    windows stepped concurrently in host threads gives the bits of one call
    over the whole run, and a second run gives them again (the benchmark's
    all-cores oracle leg relies on it)."""
    from concurrent.futures import ThreadPoolExecutor
    W, n = 8, 40_000
    hp = O.AdamW()
    G = np.stack([synth.cpu_normal_bf16(n, 2, synth.TAG_GRAD, 1, s, 0, 1e-3)
                  for s in range(W)])
    init = [synth.cpu_normal_f32(n, 2, tag, 0, 0, 0, 0.02, tag == synth.TAG_V)
            for tag in (synth.TAG_MASTER, synth.TAG_M, synth.TAG_V)]
    ref = [a.copy() for a in init]
    p_ref = O.step(G, *ref, hp, 3)
    edges = np.linspace(0, n, threads + 1).astype(int)
    for _ in range(2):
        got = [a.copy() for a in init]
        p = np.empty(n, np.uint16)

        def window(k):
            a, b = edges[k], edges[k + 1]
            views = [x[a:b] for x in got]           # contiguous slices
            p[a:b] = O.step(np.ascontiguousarray(G[:, a:b]), *views, hp, 3)

        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(window, range(threads)))
        assert np.array_equal(p, p_ref)
        for x, y in zip(got, ref):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
