"""The error of the kernels' in-place table of 2^(j/512), j < 512, by the
arithmetic the kernels use (host-only; no GPU).

The table is built as 2^(j/512) = 2^(h/16) * 2^(l/512), j = 32h + l: the 48
factors e^y (y = h * ln2/16 or l * ln2/512, each product rounded to a double)
by their Taylor series to degree 15 in Horner form with fused multiply-adds,
then one rounded product per entry.  Here each fma and product is rounded
exactly (rational arithmetic, then one rounding to binary64), so the table
is the kernels' bit for bit, and each entry is compared with e^(j ln2/512)
to 40 digits.  The fp64 exp's error budget (about 1e-14 relative from its
degree-3 polynomial) leaves room for a few ulp here; the bound asserted is
2 ulp.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

LN2O16 = float.fromhex("0x1.62e42fefa39efp-5")
LN2O512 = float.fromhex("0x1.62e42fefa39efp-10")
DEGREE = 15


def rnd(x: Fraction) -> float:
    return x.numerator / x.denominator  # int / int rounds once, to nearest


def fma(a: float, b: float, c: float) -> float:
    return rnd(Fraction(a) * Fraction(b) + Fraction(c))


def inv_factorial(k: int) -> float:
    f = 1.0
    for i in range(2, k + 1):
        f *= i
    return 1.0 / f


def factor(y: float) -> float:
    p = inv_factorial(DEGREE)
    for k in range(DEGREE - 1, -1, -1):
        p = fma(p, y, inv_factorial(k))
    return p


def test_constants_are_the_nearest_doubles():
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    assert LN2O16 == float(ln2 / 16) and LN2O512 == float(ln2 / 512)
    assert all(math.factorial(k) == int(1.0 / inv_factorial(k) + 0.5) for k in range(DEGREE + 1))


def test_table_within_two_ulp():
    getcontext().prec = 40
    ln2 = Decimal(2).ln()
    fac = [factor(rnd(Fraction(t) * Fraction(LN2O16))) for t in range(16)]
    fac += [factor(rnd(Fraction(t) * Fraction(LN2O512))) for t in range(32)]
    worst = 0.0
    for j in range(512):
        v = rnd(Fraction(fac[j >> 5]) * Fraction(fac[16 + (j & 31)]))
        exact = (ln2 * j / 512).exp()
        worst = max(worst, float(abs(Decimal(v) - exact) / Decimal(math.ulp(v))))
    assert fac[0] == 1.0 and fac[16] == 1.0
    assert worst <= 2.0, worst
