"""The E4M3 quantisers (activations, the intermediate h, RoPE) form
fl32(y / s) without a division per element: q = fl32(y * r) with
r = fl32(1 / s), the residual e = fl32(y - s q) (one fused multiply-add), then
fl32(q + e r) -- Markstein's correction step -- and an IEEE division only for
groups of four values with a quotient under 2^-9, the smallest E4M3 subnormal
(below it lie 2^-10, the one power of two that is an E4M3 rounding midpoint,
and zero).  This checks,
in exact rational arithmetic on the CPU, that the E4M3 code of the result
always equals that of the correctly rounded quotient, and that the result is
the correctly rounded quotient itself except, at most, within two ulps of a
power of two (where the residual may need one bit more than binary32 holds),
on random pairs, divisors whose significands are all ones or all zeros,
quotients next to E4M3 rounding midpoints and quotients next to powers of
two, 2^-10 among them."""
import random
from fractions import Fraction as Fr

import numpy as np

import oracle


def _rn32(x):
    """Fraction -> nearest binary32, ties to even."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fr(float(c)) - x),
                                     int(np.array([c], np.float32).view(np.uint32)[0]) & 1))


def _bits(v):
    return int(np.array([v], np.float32).view(np.uint32)[0])


def _from_bits(b):
    return np.array([b], np.uint32).view(np.float32)[0]


def test_markstein_step_gives_the_correctly_rounded_quotient():
    rng = random.Random(7)
    misses = 0
    for _ in range(20000):
        s = np.float32(np.exp(rng.uniform(-12, 2)))
        if rng.random() < 0.2:
            s = _from_bits((_bits(s) & 0xFF800000) | rng.choice([0x7FFFFF, 0, 0x7FFFFE, 1, 0x400000]))
        y = np.float32(rng.gauss(0, 1) * float(s) * rng.choice([1, 30, 300, 448]))
        if rng.random() < 0.3:
            m = rng.choice([17 / 16, 1.125, 272.0, 432.0, 0.28125, 13.5])
            y = _from_bits(_bits(np.float32(m * float(s))) + rng.randint(-3, 3))
        Y, S = Fr(float(y)), Fr(float(s))
        r = _rn32(1 / S)
        q0 = _rn32(Y * Fr(float(r)))
        e = _rn32(Y - S * Fr(float(q0)))
        q1 = _rn32(Fr(float(e)) * Fr(float(r)) + Fr(float(q0)))
        want = _rn32(Y / S)
        clamp = lambda v: float(min(max(v, -448.0), 448.0))  # noqa: E731
        assert oracle.e4m3_from_f32(clamp(q1)) == oracle.e4m3_from_f32(clamp(want)), (y, s)
        if q1 != want:
            p2 = 2.0 ** np.round(np.log2(abs(float(want))))
            assert abs(float(want) - p2) <= 2 * abs(float(np.spacing(np.float32(p2)))), (y, s, q1, want)
            misses += 1
    assert misses <= 20000 // 1000


def _kernel_quotient(y, s):
    """The kernels' quotient (common.hpp e4m3_codes4 before the clamp), in
    exact arithmetic, one value at a time: the correction step, the IEEE
    quotient under 2^-9 in magnitude.  (The kernels
    divide all four values of a group that holds such a quotient; the others
    then take the correctly rounded quotient, whose code is the same.)"""
    Y, S = Fr(float(y)), Fr(float(s))
    r = _rn32(1 / S)
    q0 = _rn32(Y * Fr(float(r)))
    e = _rn32(Y - S * Fr(float(q0)))
    q = _rn32(Fr(float(e)) * Fr(float(r)) + Fr(float(q0)))
    if not abs(float(q)) >= 2.0 ** -9:
        q = _rn32(Y / S)
        if float(q) == 0.0:
            q = np.float32(np.copysign(0.0, float(y)))  # IEEE: the sign of y / s
    return np.float32(q)


def test_quotient_next_to_powers_of_two_and_the_subnormal_midpoint():
    """Quotients within two ulps of 2^-10 (an E4M3 midpoint: ties go to the
    even code 0), 2^-9, 2^-3 and 1, over divisors with random significands:
    the code always equals that of the correctly rounded quotient; -0 keeps
    its sign."""
    rng = random.Random(11)
    for p in (2.0 ** -10, 2.0 ** -9, 2.0 ** -3, 1.0):
        for _ in range(1500):
            s = _from_bits((rng.randrange(100, 140) << 23) | rng.randrange(0, 1 << 23))
            y0 = _bits(np.float32(p * float(s)))
            for k in (-2, -1, 0, 1, 2):
                y = _from_bits(y0 + k)
                want = _rn32(Fr(float(y)) / Fr(float(s)))
                got = _kernel_quotient(y, s)
                assert oracle.e4m3_from_f32(float(got)) == oracle.e4m3_from_f32(float(want)), (p, y, s)
    s = np.float32(0.37)
    assert _bits(_kernel_quotient(np.float32(-0.0), s)) == 0x80000000
    assert oracle.e4m3_from_f32(float(_kernel_quotient(np.float32(-0.0), s))) == 0x80
