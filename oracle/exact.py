"""Exact-arithmetic RMSNorm for tiny inputs -- TEST INFRASTRUCTURE ONLY.

An independent second reference, used to pin the fp64 C oracle: every input
float is converted to an exact rational, the sum of squares and the mean are
exact rationals, and the square root and the division are done in decimal
arithmetic with 60 significant digits. For tiny rows (pure-Python loops) it
gives the RMSNorm of Eq. 1 of the SwiftQK technical review ("Prerequisites")
to far beyond fp64 precision.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

_DIGITS = 60


def _dec(fr):
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def sum_of_squares(values):
    """Exact sum of squares of a sequence of floats, as a Fraction."""
    total = Fraction(0)
    for v in values:
        f = Fraction(float(v))
        total += f * f
    return total


def rmsnorm_row(x, gamma, eps):
    """Eq. 1 for one row, exactly up to 60 digits: returns a list of Decimals.

    eps is taken as the exact value of the float given (pass the float32
    value the GPU library receives).
    """
    getcontext().prec = _DIGITS
    H = len(x)
    mean_plus_eps = sum_of_squares(x) / H + Fraction(float(eps))
    rms = _dec(mean_plus_eps).sqrt()
    return [_dec(Fraction(float(xj))) / rms * _dec(Fraction(float(gj)))
            for xj, gj in zip(x, gamma)]


def inverse_rms(x, eps, H_total=None):
    """1 / sqrt(sum(x^2)/H_total + eps) as a Decimal (Eq. 6); H_total defaults
    to len(x)."""
    getcontext().prec = _DIGITS
    H = len(x) if H_total is None else H_total
    return 1 / _dec(sum_of_squares(x) / H + Fraction(float(eps))).sqrt()
