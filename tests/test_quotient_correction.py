"""The FP8 cache write divides each element by its row scale s through the
correctly rounded reciprocal r = 1/s and one correction step (Markstein):

    q  = RN(x r),   e = x - q s (exact in an FMA),   q' = RN(q + e r)

instead of one IEEE division per element.  This checks, in exact rational
arithmetic on the CPU, that q' equals the correctly rounded float32 quotient
RN(x / s) for the scales the write produces (s = amax / 448) and for x drawn
from every binade the 16-bit inputs reach, including quotients placed next to
the midpoints where E4M3 rounding is decided -- the cases where a last-bit
error would change a code.
"""

from fractions import Fraction

import numpy as np

F32 = np.float32


def rn32(v: Fraction) -> float:
    """v rounded to the nearest float32, ties to even (normal range)."""
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scale = Fraction(2) ** (23 - e)           # 24 significant bits
    m = a * scale
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) / scale)


def fma32(a, b, c) -> float:
    return rn32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def corrected_quotient(x, s) -> float:
    r = F32(F32(1.0) / F32(s))                 # IEEE division: correctly rounded
    q = F32(F32(x) * r)
    e = fma32(-float(q), s, x)
    return float(np.copysign(fma32(e, float(r), float(q)), x))


def test_corrected_quotient_is_correctly_rounded():
    rng = np.random.default_rng(7)
    cases = 0
    for _ in range(300):
        amax = F32(abs(rng.standard_normal()) * 2.0 ** rng.integers(-12, 9))
        if amax == 0:
            continue
        s = F32(amax / F32(448))
        xs = [F32(v) for v in rng.uniform(-1, 1, 40) * float(amax)] + [amax, -amax, F32(0), F32(-0.0)]
        # quotients placed at and next to E4M3 rounding midpoints (m + 1/2) * 2^(k-3)
        for _ in range(20):
            k = int(rng.integers(-6, 9))
            m = int(rng.integers(8, 16))
            mid = (m + 0.5) * 2.0 ** (k - 3)
            base = F32(mid * float(s))
            for dx in (-2, -1, 0, 1, 2):
                v = base
                for _ in range(abs(dx)):
                    v = F32(np.nextafter(v, F32(np.inf) if dx > 0 else F32(-np.inf)))
                xs.append(v)
        for x in xs:
            if abs(float(x)) > float(amax):
                continue
            want = rn32(Fraction(float(x)) / Fraction(float(s))) if x != 0 else float(np.copysign(0.0, x))
            got = corrected_quotient(x, s)
            assert got == want and np.signbit(got) == np.signbit(want), (float(x), float(s), got, want)
            cases += 1
    assert cases > 10000
