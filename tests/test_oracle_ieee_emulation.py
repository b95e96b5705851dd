"""Pin of the step oracle's floating-point semantics against exact rational
arithmetic.

The readings of the pages' step (reduce-scatter with SUM then the rank-local
AdamW update: CS336 lecture 8 notes, "Code example: ZeRO-1"; AdamW per the
DDP-to-ZeRO blog, section 3.3) fix each statement as one IEEE binary32
operation rounded once to nearest-even: the sum from the first rank's value
in rank order, the division by W, the two moment updates, the correctly
rounded square root, the divide, the decoupled decay, and the bf16 copy
rounded to nearest-even.  Here every such operation is carried out on exact
fractions (Python's Fraction) and rounded to binary32 by integer arithmetic,
so the result does not depend on any floating-point unit: a C oracle built
with contracted multiply-adds, extended intermediates, an approximate square
root or a reciprocal in place of a divide would differ from it in the last
bit.  The per-call constants are taken, as the reading states, from double
precision rounded once to fp32 (computed here with Python floats).
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import step as O

EMIN, MBITS = -126, 24          # binary32: smallest normal exponent, digits


def _round_mag(a: Fraction, bits: int) -> Fraction:
    """Nearest binary number to a > 0 with `bits` significant digits and
    the binary32 exponent range below (subnormals at 2^-149), ties to
    even; the overflow threshold is left to the caller."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    quantum = Fraction(2) ** (max(e, EMIN) - (bits - 1))
    q, r = divmod(a.numerator * quantum.denominator,
                  a.denominator * quantum.numerator)
    twice = 2 * r
    den = a.denominator * quantum.numerator
    if twice > den or (twice == den and q % 2):
        q += 1
    return q * quantum


def r32(x: Fraction) -> Fraction:
    if x == 0:
        return Fraction(0)
    y = _round_mag(abs(x), MBITS)
    if y >= Fraction(2) ** 128:
        raise OverflowError("outside the finite range of this pin")
    return y if x > 0 else -y


def sqrt32(x: Fraction) -> Fraction:
    """Correctly rounded binary32 square root of x >= 0: the candidates
    around an integer-square-root approximation, chosen by comparing x with
    the squares of their midpoints (exact)."""
    if x == 0:
        return Fraction(0)
    K = 200
    n = x.numerator * (1 << (2 * K)) // x.denominator
    approx = Fraction(math.isqrt(n), 1 << K)
    y = r32(approx)
    f = np.float32(float(y))
    cands = sorted({float(np.nextafter(f, np.float32(0))), float(f),
                    float(np.nextafter(f, np.float32(np.inf)))})
    cands = [Fraction(c) for c in cands if c > 0]
    best = cands[0]
    for c in cands[1:]:
        mid = (best + c) / 2
        if x > mid * mid:
            best = c
        elif x == mid * mid:                     # tie: the even significand
            bits = np.float32(float(c)).view(np.uint32)
            if bits % 2 == 0:
                best = c
    return best


def bf16_bits(x: Fraction) -> int:
    """Nearest bf16 (8 significant digits, binary32 exponent range) to the
    binary32 value x, ties to even, as its 16-bit pattern."""
    y = Fraction(0) if x == 0 else _round_mag(abs(x), 8)
    if x < 0:
        y = -y
    f = np.float32(float(y))
    return int(f.view(np.uint32)) >> 16


def f32(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def consts(hp, t):
    """The per-call constants: the fp32 hyper-parameters widened to double,
    each constant evaluated there and rounded once to binary32."""
    b1, b2, lr, wd, eps = (float(np.float32(x)) for x in
                           (hp.beta1, hp.beta2, hp.lr, hp.weight_decay,
                            hp.eps))
    return dict(b1=f32(b1), b2=f32(b2), om1=f32(1.0 - b1), om2=f32(1.0 - b2),
                ss=f32(lr / (1.0 - b1 ** t)),
                bc2s=f32(math.sqrt(1.0 - b2 ** t)),
                dec=f32(1.0 - lr * wd), eps=f32(eps))


def emulate(Gcol, master, m, v, hp, t, mistake=None):
    """One element of the step in exact arithmetic, each statement rounded
    once to binary32; returns (master, m, v, bf16 bits).  `mistake` names a
    plausible wrong evaluation, used only to show that the pin would catch
    it."""
    W = len(Gcol)
    c = consts(hp, t)
    b1, b2, om1, om2 = c["b1"], c["b2"], c["om1"], c["om2"]
    ss, bc2s, dec, eps = c["ss"], c["bc2s"], c["dec"], c["eps"]
    G = [Fraction(float(O.bf16_to_f32(np.uint16(x)))) for x in Gcol]
    if mistake == "sum in reverse rank order":
        G = G[::-1]
    acc = G[0]
    for x in G[1:]:
        acc = acc + x if mistake == "exact sum" else r32(acc + x)
    if mistake == "mean as a product with 1/W":
        g = r32(acc * r32(Fraction(1, W)))
    else:
        g = r32(acc / W)
    if mistake == "fused moment update":
        mi = r32(r32(b1 * m) + om1 * g)
    else:
        mi = r32(r32(b1 * m) + r32(om1 * g))
    vi = r32(r32(b2 * v) + r32(om2 * r32(g * g)))
    if mistake == "bias correction as a product":
        den = r32(r32(sqrt32(vi) * r32(1 / bc2s)) + eps)
    else:
        den = r32(r32(sqrt32(vi) / bc2s) + eps)
    if mistake == "update as a product with 1/den":
        upd = r32(mi * r32(1 / den))
    else:
        upd = r32(mi / den)
    if mistake == "fused decay":
        th = r32(master * dec - r32(ss * upd))
    else:
        th = r32(r32(master * dec) - r32(ss * upd))
    if mistake == "bf16 by truncation":
        bits = int(np.float32(float(th)).view(np.uint32)) >> 16
        return th, mi, vi, bits
    return th, mi, vi, bf16_bits(th)


@pytest.mark.parametrize("W,sigma,kw", [
    (1, 1e-3, {}),
    (3, 1e-3, {}),
    (8, 1.0, {}),
    (5, 1e-6, dict(eps=1e-6)),                  # eps comparable to sqrt(v)
    (4, 1e-2, dict(lr=0.05, weight_decay=0.3, beta1=0.8, beta2=0.9)),
    (6, 1e-4, dict(spread=16.0)),             # sums that round, rank order
    (3, 1e-21, {}),                           # g*g and v in the subnormals
])
def test_step_equals_exact_per_operation_rounding(W, sigma, kw):
    n = 300
    base = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    base.update(kw)
    spread = base.pop("spread", 1.0)
    hp = O.AdamW(**base)
    master = synth.cpu_normal_f32(n, 1, synth.TAG_MASTER, 0, 0, 0, 0.02)
    m = (synth.cpu_normal_f32(n, 2, synth.TAG_MASTER, 0, 0, 0, 1.0)
         * np.float32(sigma)).astype(np.float32)
    v = np.abs(synth.cpu_normal_f32(n, 3, synth.TAG_MASTER, 0, 0, 0, 1.0)
               * np.float32(sigma * sigma)).astype(np.float32)
    em = [(Fraction(float(a)), Fraction(float(b)), Fraction(float(c)))
          for a, b, c in zip(master, m, v)]
    for t in (1, 2, 7):
        G = np.stack([synth.cpu_normal_bf16(n, 4, synth.TAG_GRAD, t, s, 0,
                                            sigma * spread ** s)
                      for s in range(W)])
        p16 = O.step(G, master, m, v, hp, t)
        for i in range(n):
            th, mi, vi, pb = emulate(G[:, i], *em[i], hp, t)
            em[i] = (th, mi, vi)
            where = f"W={W} t={t} i={i}"
            assert Fraction(float(master[i])) == th, where
            assert Fraction(float(m[i])) == mi, where
            assert Fraction(float(v[i])) == vi, where
            assert int(p16[i]) == pb, where


MISTAKES = ["sum in reverse rank order", "exact sum",
            "mean as a product with 1/W", "fused moment update",
            "bias correction as a product",
            "update as a product with 1/den", "fused decay",
            "bf16 by truncation"]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_pin_catches_a_plausible_mistake(mistake):
    """The pin is sharp: each wrong evaluation above, computed just as
    exactly, disagrees with the oracle on some element of one step."""
    W, n = 6, 400
    hp = O.AdamW(lr=0.05, beta1=0.9, beta2=0.95, eps=1e-8,
                 weight_decay=0.3)
    master = synth.cpu_normal_f32(n, 5, synth.TAG_MASTER, 0, 0, 0, 1.0)
    m = synth.cpu_normal_f32(n, 6, synth.TAG_MASTER, 0, 0, 0, 1e-2)
    v = synth.cpu_normal_f32(n, 7, synth.TAG_MASTER, 0, 0, 0, 1e-4,
                             absval=True)
    # ranks' gradients four binary orders apart, so that the fp32 sum of
    # bf16 values rounds and its order shows
    G = np.stack([synth.cpu_normal_bf16(n, 8, synth.TAG_GRAD, 3, s, 0,
                                        1e-4 * 16.0 ** s) for s in range(W)])
    before = [(Fraction(float(a)), Fraction(float(b)), Fraction(float(c)))
              for a, b, c in zip(master, m, v)]
    p16 = O.step(G, master, m, v, hp, 3)
    differs = 0
    for i in range(n):
        right = emulate(G[:, i], *before[i], hp, 3)
        wrong = emulate(G[:, i], *before[i], hp, 3, mistake)
        got = (Fraction(float(master[i])), Fraction(float(m[i])),
               Fraction(float(v[i])), int(p16[i]))
        assert got == right, i
        differs += wrong != got
    assert differs > 0, mistake


def bf16_value(bits) -> Fraction:
    return Fraction(float(O.bf16_to_f32(np.uint16(bits))))


@pytest.mark.parametrize("W", [1, 3, 8])
def test_pure_bf16_step_equals_exact_per_operation_rounding(W):
    """The step without an fp32 master: the same statements on the bf16
    parameter widened to fp32, the result rounded back to bf16 nearest-even
    in place (the pure-bf16 reading of the DDP-to-ZeRO blog's mixed
    precision, section 3.3)."""
    n = 300
    hp = O.AdamW(lr=1e-2, weight_decay=0.1)
    p = O.bf16_round(synth.cpu_normal_f32(n, 11, synth.TAG_MASTER, 0, 0, 0,
                                          0.02))
    m = synth.cpu_normal_f32(n, 12, synth.TAG_MASTER, 0, 0, 0, 1e-3)
    v = synth.cpu_normal_f32(n, 13, synth.TAG_MASTER, 0, 0, 0, 1e-6,
                             absval=True)
    em = [(bf16_value(a), Fraction(float(b)), Fraction(float(c)))
          for a, b, c in zip(p, m, v)]
    for t in (1, 2, 5):
        G = np.stack([synth.cpu_normal_bf16(n, 14, synth.TAG_GRAD, t, s, 0,
                                            1e-3 * 16.0 ** s)
                      for s in range(W)])
        O.step_bf16(G, p, m, v, hp, t)
        for i in range(n):
            _, mi, vi, pb = emulate(G[:, i], *em[i], hp, t)
            em[i] = (bf16_value(pb), mi, vi)
            where = f"W={W} t={t} i={i}"
            assert int(p[i]) == pb, where
            assert Fraction(float(m[i])) == mi, where
            assert Fraction(float(v[i])) == vi, where


@pytest.mark.parametrize("k", [2, 3, 6])
def test_accumulation_equals_exact_per_operation_rounding(k):
    """Gradient accumulation: the fp32 sum of the k micro-batch gradients
    in micro-batch order, one rounding per addition, divided by k with one
    rounding, then bf16 nearest-even (podcast summary of "Training at
    thousands of GPUs", glossary; DDP-to-ZeRO blog, section 3.3)."""
    n = 2000
    G = np.stack([synth.cpu_normal_bf16(n, 15, synth.TAG_GRAD, j, 0, 0,
                                        1e-4 * 16.0 ** j) for j in range(k)])
    out = O.accumulate(G)
    for i in range(n):
        acc = bf16_value(G[0, i])
        for j in range(1, k):
            acc = r32(acc + bf16_value(G[j, i]))
        assert int(out[i]) == bf16_bits(r32(acc / k)), (k, i)
