"""The RoPE quantiser forms fl32(y / s) without a division per element:
q = fl32(y * r) with r = fl32(1 / s), the residual e = fl32(y - s q) (one
fused multiply-add), then fl32(q + e r) -- Markstein's correction step.  This
checks, in exact rational arithmetic on the CPU, that the E4M3 code of the
result always equals that of the correctly rounded quotient, and that the
result is the correctly rounded quotient itself except, at most, within two
ulps of a power of two (where the residual may need one bit more than binary32
holds; powers of two are E4M3 values, never rounding midpoints), on random
pairs, divisors whose significands are all ones or all zeros and quotients
next to E4M3 rounding midpoints."""
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
