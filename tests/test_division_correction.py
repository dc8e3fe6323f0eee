"""The V pass divides every residual by its channel's scale with one reciprocal per channel and
two FMA corrections instead of a division per element.  Emulated here in exact rational
arithmetic with float32 rounding at each step (each FMA rounded once), the result must equal the
correctly rounded quotient for random and for adversarial operands (divisor significands of all
ones, quotients at binade edges and on E4M3 rounding boundaries)."""
from fractions import Fraction

import numpy as np


def rn32(v: Fraction) -> Fraction:
    """Round an exact rational to the nearest float32 value (ties to even); normal range only."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def f(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def qdiv(x: Fraction, s: Fraction) -> Fraction:
    y = rn32(1 / s)
    q = rn32(x * y)
    q = rn32((x - q * s) * y + q)          # fmaf(fmaf(-q, s, x), y, q): the inner FMA is exact
    return rn32(rn32(x - q * s) * y + q)


def test_corrected_reciprocal_division_is_correctly_rounded():
    rng = np.random.default_rng(0)
    cases = []
    for _ in range(4000):
        s = f(rng.uniform(0.001, 4.0))
        x = f(rng.uniform(-448.0, 448.0) * float(s))
        cases.append((x, s))
    # divisors whose significand is all ones or one below a power of two
    for k in range(-12, 4):
        for s in (Fraction(2) ** k * (2 - Fraction(1, 2 ** 23)), Fraction(2) ** k * (1 + Fraction(1, 2 ** 23))):
            for _ in range(60):
                cases.append((f(rng.uniform(-448.0, 448.0) * float(s)), s))
    # quotients next to E4M3 rounding midpoints and to binade edges
    for _ in range(1500):
        s = f(rng.uniform(0.01, 2.0))
        e = int(rng.integers(-6, 8))
        m = int(rng.integers(8, 16))
        mid = Fraction(2 * m + 1, 16) * Fraction(2) ** e          # halfway between two E4M3 codes
        for t in (mid, Fraction(2) ** e):
            x = rn32(t * s)
            for dx in (-2, -1, 0, 1, 2):
                cases.append((x + dx * Fraction(2) ** (x.numerator.bit_length() - x.denominator.bit_length() - 24), s))
    bad = [(x, s) for x, s in cases if x != 0 and qdiv(rn32(x), s) != rn32(rn32(x) / s)]
    assert not bad, bad[:3]
