"""Exact rational arithmetic used to pin the oracle (test helper, not part of it).

Everything here works on ``fractions.Fraction`` and Python integers: no
floating-point operation takes part in a rounding decision, so these helpers
cannot share a rounding mistake with the oracle's C code or with numpy.
"""
from __future__ import annotations

from fractions import Fraction


def f16_bits_to_fraction(bits: int) -> Fraction:
    """Exact value of a finite IEEE binary16 bit pattern."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    assert e != 31, "not finite"
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(m + 1024) * Fraction(2) ** (e - 25)


def f32_bits_to_fraction(bits: int) -> Fraction:
    sign = -1 if bits & 0x80000000 else 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    assert e != 255
    if e == 0:
        return sign * Fraction(m) * Fraction(2) ** -149
    return sign * Fraction(m + (1 << 23)) * Fraction(2) ** (e - 150)


def _floor_log2(r: Fraction) -> int:
    """Largest e with 2**e <= r, for r > 0."""
    e = r.numerator.bit_length() - r.denominator.bit_length()
    if Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    return e


def _round_half_even(r: Fraction) -> int:
    n = r.numerator // r.denominator
    rem = r - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def round_to_binary(r: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round ``r`` to the nearest value of a binary format with ``mant_bits``
    stored fraction bits, minimum normal exponent ``emin`` and maximum exponent
    ``emax``; ties to even; overflow returns +-inf as a float."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = max(_floor_log2(a), emin)           # subnormals share emin's quantum
    quantum = Fraction(2) ** (e - mant_bits)
    n = _round_half_even(a / quantum)
    v = n * quantum
    if v >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * v


def to_f32(r: Fraction) -> Fraction:
    return round_to_binary(r, 23, -126, 127)


def to_f16(r: Fraction) -> Fraction:
    return round_to_binary(r, 10, -14, 15)


def round_half_away(r: Fraction) -> int:
    a = abs(r)
    n = a.numerator // a.denominator
    if a - n >= Fraction(1, 2):
        n += 1
    return n if r >= 0 else -n


def quantize_exact(xs: list[Fraction], qmax: int):
    """The quantizer rule written with exact arithmetic: s = fl32(amax/qmax),
    q = clamp(round_half_away(fl32(x/s)), -qmax, qmax)."""
    amax = max((abs(x) for x in xs), default=Fraction(0))
    if amax == 0:
        return Fraction(0), [0] * len(xs)
    s = to_f32(amax / qmax)
    codes = []
    for x in xs:
        t = to_f32(x / s)
        q = max(-qmax, min(qmax, round_half_away(t)))
        codes.append(q)
    return s, codes
