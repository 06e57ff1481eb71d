"""Exact rational rounding helpers for the oracle's pins.

These are written from the IEEE-754 binary formats (round to nearest, ties to
even) with Python integers and fractions.Fraction; they share nothing with the
oracle's numpy code, so agreement between the two is evidence, not an echo.
"""

from __future__ import annotations

from fractions import Fraction


def _round_half_even(q: Fraction) -> int:
    """Nearest integer to a non-negative rational, ties to even."""
    n, r = divmod(q.numerator, q.denominator)
    twice = 2 * r
    if twice > q.denominator or (twice == q.denominator and n % 2 == 1):
        n += 1
    return n


def round_binary(q: Fraction, mant_bits: int, emin: int, emax: int, saturate_to=None) -> Fraction:
    """Round q to a binary format with ``mant_bits`` fraction bits, smallest
    normal exponent ``emin`` and largest exponent ``emax`` (RNE).  Overflow
    returns None, or ``saturate_to`` when given."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)  # subnormals share the quantum of the smallest binade
    quantum = Fraction(2) ** (e - mant_bits)
    n = _round_half_even(a / quantum)
    v = n * quantum
    max_finite = (2 - Fraction(2) ** -mant_bits) * Fraction(2) ** emax
    if v > max_finite:
        if saturate_to is None:
            return None
        v = Fraction(saturate_to)
    return sign * v


def to_f32(q: Fraction) -> Fraction:
    return round_binary(q, 23, -126, 127)


def to_bf16(q: Fraction) -> Fraction:
    return round_binary(q, 7, -126, 127)


def e4m3_code(q: Fraction, negative: bool) -> int:
    """E4M3 (OCP FN) code of a rational by exact RNE on the format's grid,
    saturating to 448; ``negative`` carries the sign (so -0 can be expressed)."""
    v = round_binary(abs(q), 3, -6, 20)  # wide exponent range: overflow handled below
    if v > 448:
        v = Fraction(448)
    if v == 0:
        code = 0
    elif v >= Fraction(1, 64):
        e = v.numerator.bit_length() - v.denominator.bit_length()
        if Fraction(2) ** e > v:
            e -= 1
        m = (v / Fraction(2) ** e - 1) * 8
        assert m.denominator == 1
        code = ((e + 7) << 3) | int(m)
    else:
        m = v / Fraction(1, 512)
        assert m.denominator == 1
        code = int(m)
    return code | (0x80 if negative else 0)


def f32_fraction(x) -> Fraction:
    """Exact rational value of a finite float (numpy float32 or Python float)."""
    return Fraction(float(x))
