"""Exact rational rounding to IEEE binary formats, for pins.

Independent of numpy's bit tricks: a value is rounded by taking its exact
rational value, finding its binade, and rounding the scaled significand to the
nearest integer with ties to even.  Used to re-derive bf16 and fp32 results of
tiny problems by brute force.
"""
from fractions import Fraction
import math

_FMT = {
    # name: (significand bits incl. the hidden one, min normal exponent, max exponent)
    "fp32": (24, -126, 127),
    "bf16": (8, -126, 127),
}


def _floor_log2(q: Fraction) -> int:
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    if (n << max(0, -e)) < (d << max(0, e)):
        e -= 1
    return e


def round_to(q, fmt: str) -> float:
    """Round a finite real (Fraction/int/float) to `fmt`, ties to even.
    Returns a Python float (inf on overflow)."""
    p, emin, emax = _FMT[fmt]
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    k = a / quantum
    fl = k.numerator // k.denominator
    rem = k - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    max_finite = (Fraction(2) - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > max_finite:
        return sign * math.inf
    return sign * float(r)


def _exact(x) -> Fraction:
    if isinstance(x, (int, Fraction)):
        return Fraction(x)
    return Fraction(float(x))  # numpy scalars and floats are exact binary values


def fp32(x) -> float:
    return round_to(_exact(x), "fp32")


def bf16(x) -> float:
    return round_to(_exact(x), "bf16")


def fp32_sqrt(x) -> float:
    """Correctly rounded fp32 square root of a non-negative finite value
    (ties to even), from integer square roots of the exact rational."""
    q = _exact(x)
    if q < 0:
        raise ValueError("negative")
    if q == 0:
        return 0.0
    p, emin, _ = _FMT["fp32"]
    e = max(_floor_log2(q) // 2, emin)        # binade of sqrt(q)
    quantum = Fraction(2) ** (e - p + 1)
    k2 = q / (quantum * quantum)               # (sqrt(q) / quantum)^2
    fl = math.isqrt(k2.numerator // k2.denominator)
    half = (Fraction(2 * fl + 1, 2)) ** 2
    if k2 > half or (k2 == half and fl % 2 == 1):
        fl += 1
    return float(fl * quantum)
