"""Pins of the gradient-accumulation oracle (oracle.step.accumulate: k
micro-batch bf16 gradients summed in fp32 in order, divided by k, rounded
to bf16) against the mathematics: k = 1 is the identity, sums of small
integers are exact, the order of the sum is fixed, and a float64 evaluation
agrees within the roundings of the formula."""

import numpy as np
import pytest

import synth
from oracle import step as O


def grads(k, n, sigma=1e-3, seed=0):
    return np.stack([synth.cpu_normal_bf16(n, seed, synth.TAG_GRAD, j, 0, 0,
                                           sigma) for j in range(k)])


def test_one_micro_batch_is_the_identity():
    G = grads(1, 4096)
    assert np.array_equal(O.accumulate(G), G[0])
    # every finite bf16 pattern too
    allp = np.arange(1 << 16, dtype=np.uint16)
    finite = (allp & 0x7f80) != 0x7f80
    assert np.array_equal(O.accumulate(allp[None, finite]), allp[finite])


def test_small_integers_are_exact():
    # integers up to 256 are exact in bf16; their sums and power-of-two
    # means are exact in fp32 and in bf16 when the mean stays an integer
    rng = np.random.default_rng(0)
    k = 4
    ints = rng.integers(-64, 65, (k, 1000)) * 4           # multiples of k
    G = O.bf16_round(ints.astype(np.float32))
    want = O.bf16_round((ints.sum(0) / k).astype(np.float32))
    assert np.array_equal(O.accumulate(G), want)
    assert np.array_equal(O.bf16_to_f32(want), ints.sum(0) / k)


def test_fixed_order_of_the_sum():
    # (a + b) + c differs from a + (b + c) for a = 1, b = c = 2^-24: fp32 sum
    # in order gives 1 (each tiny term is lost); the pages' serial addition
    # fixes the order
    one, tiny = 0x3f80, 0x3380                     # 1.0, 2^-24 in bf16
    G = np.array([[one], [tiny], [tiny]], np.uint16)
    # mean = 1/3 in fp32 then bf16: computed from acc = 1.0 exactly
    want = O.bf16_round(np.array([np.float32(1.0) / np.float32(3)]))
    assert np.array_equal(O.accumulate(G), want)
    G2 = np.array([[tiny], [tiny], [one]], np.uint16)
    acc = np.float32(2.0 ** -24) + np.float32(2.0 ** -24) + np.float32(1.0)
    assert np.array_equal(O.accumulate(G2),
                          O.bf16_round(np.array([acc / np.float32(3)])))


@pytest.mark.parametrize("k", [2, 3, 8])
def test_float64_agrees_within_the_roundings(k):
    G = grads(k, 8192, sigma=1.0, seed=k)
    exact = O.bf16_to_f32(G).astype(np.float64).sum(0) / k
    got = O.bf16_to_f32(O.accumulate(G)).astype(np.float64)
    # fp32 sum of k terms + one division: relative error << one bf16 ulp,
    # so the result is the bf16 rounding of the exact mean or a neighbour
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64) \
        * 2 ** 16
    assert np.all(np.abs(got - exact) <= ulp + 1e-30)


def _round_half_even(fr, bits):
    """The binary floating-point number nearest to the positive rational fr
    with `bits` significant bits (ties to even), as a Fraction: exact
    integer arithmetic, no floating point."""
    from fractions import Fraction
    e = fr.numerator.bit_length() - fr.denominator.bit_length()
    if Fraction(2) ** e > fr:
        e -= 1                                   # 2^e <= fr < 2^(e+1)
    scale = Fraction(2) ** (bits - 1 - e)
    m = fr * scale                               # in [2^(bits-1), 2^bits)
    q, r = divmod(m.numerator, m.denominator)
    twice = 2 * r
    if twice > m.denominator or (twice == m.denominator and q % 2):
        q += 1
    return Fraction(q) / scale


def _tie_columns(k, n, rng):
    """n columns of k bf16-exact integers whose sum is k*q with q odd in
    [257, 509]: the exact mean lies halfway between two neighbouring bf16
    values (spaced 2 there), so the bf16 result is decided by the fp32
    quotient being exact."""
    cols = []
    while len(cols) < n:
        q = 2 * int(rng.integers(129, 255)) + 1
        big = [2 * int(x) for x in rng.integers(128, 256, k - 1)]
        r = k * q - sum(big)
        if 1 <= r <= 256:                        # exact in bf16 as well
            cols.append(big + [r])
    return np.array(cols, np.int64).T


@pytest.mark.parametrize("k", [3, 5, 7])
def test_division_by_k_is_correctly_rounded(k):
    """Integer gradients (exact in bf16, sums exact in fp32) divided by k,
    not a power of two: the oracle's bf16 result equals the exact quotient
    rounded to fp32 (24 bits) and then to bf16 (8 bits), both to nearest
    even, computed here with exact rational arithmetic.  Half the columns
    put the exact mean halfway between two bf16 values, where a quotient
    that is not correctly rounded in fp32 tips the bf16 result the other
    way (a multiply by fp32 1/7 does so in 284 of these 1000 columns; at
    k = 3 and 5 that product happens to round to the exact quotient)."""
    from fractions import Fraction
    rng = np.random.default_rng(k)
    ints = np.concatenate([rng.integers(1, 257, (k, 1000)),
                           _tie_columns(k, 1000, rng)], axis=1)
    G = O.bf16_round(ints.astype(np.float32))
    assert np.array_equal(O.bf16_to_f32(G), ints)       # inputs are exact
    got = O.bf16_to_f32(O.accumulate(G))
    for s, g in zip(ints.sum(0), got):
        q32 = _round_half_even(Fraction(int(s), k), 24)
        want = _round_half_even(q32, 8)
        assert Fraction(float(g)) == want, (s, k, float(g), float(want))
