"""Host checks of a piece of floating-point arithmetic that the row-strip
statistics pass (k_factored.hip, k_f_strip) relies on.

Each row's mean is fl32(sum / C) of a double row sum. The kernel forms the
double quotient without a division: q0 = RN(sum * y) with y = RN(1/C), the
exact residual r = sum - C q0 (one fma), and RN(q0 + r y) (one fma). By
Markstein's theorem (Markstein, "Computation of elementary functions on the
IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990; restated in
Muller et al., Handbook of Floating-Point Arithmetic, on division with an
fma) the result is the correctly rounded quotient, the same double as an
IEEE division, whenever y is within half an ulp of 1/C and q0 within one ulp
of sum / C. The second condition holds when y's relative error is at most
2^-54, which these tests check for every column count the pass accepts
(C = m * 512, m = 1..24), and the quotient itself is checked against Python's
correctly rounded division on random and edge-case sums, with every fma
emulated exactly in rationals.
"""
import math
import random
from fractions import Fraction

import pytest

STRIP_COLUMNS = [m * 512 for m in range(1, 25)]


def fma(a, b, c):
    """a * b + c rounded once to double (exact rational arithmetic)."""
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def corrected_quotient(s, C):
    y = 1.0 / C
    q0 = s * y
    r = fma(-float(C), q0, s)
    return fma(r, y, q0)


@pytest.mark.parametrize("C", STRIP_COLUMNS)
def test_reciprocal_within_2_pow_minus_54(C):
    y = 1.0 / C
    assert abs(1 - Fraction(C) * Fraction(y)) <= Fraction(1, 2 ** 54)


@pytest.mark.parametrize("C", STRIP_COLUMNS)
def test_corrected_quotient_equals_division(C):
    rng = random.Random(C)
    sums = [rng.uniform(1.0, 2.0) * 2.0 ** rng.randint(-150, 150) for _ in range(2000)]
    for e in (-149, -60, 0, 1, 37, 200):
        b = 2.0 ** e
        sums += [b, math.nextafter(b, 0.0), math.nextafter(b, math.inf), math.nextafter(2 * b, 0.0)]
        sums += [C * b * (1 + k * 2.0 ** -52) for k in (-3, -1, 1, 2, 5)]
        sums += [C * b * rng.randint(1, 1 << 20) for _ in range(20)]
    for s in sums:
        assert corrected_quotient(s, C) == s / C, (s, C)


def test_plain_product_alone_is_not_enough():
    """Without the correction RN(sum * RN(1/C)) misses the IEEE quotient on
    some sums, so the residual step is what makes the mean exact."""
    C = 3 * 512
    rng = random.Random(7)
    sums = [rng.uniform(1.0, 2.0) for _ in range(20000)]
    assert any(s * (1.0 / C) != s / C for s in sums)
