"""Exact-arithmetic helpers for the oracle pins, written independently of oracle.c.

Everything here works on Python integers and fractions.Fraction, so a rounding
decision made here cannot inherit a mistake from the C oracle's double or
long-double arithmetic.
"""
from __future__ import annotations

import struct
from fractions import Fraction
from typing import Union

Number = Union[int, Fraction]


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern (sign, 8-bit exponent, 7-bit fraction)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    assert e != 0xFF, "inf/nan"
    if e == 0:
        mag = Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    else:
        mag = (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))
    return sign * mag


def floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    assert a > 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def rn_bf16_bits(v: Number, negative_zero: bool = False) -> int:
    """Round an exact value to the nearest bf16 (ties to even), return its bit pattern."""
    v = Fraction(v)
    if v == 0:
        return 0x8000 if negative_zero else 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = max(floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 7)
    n = round_half_even(a / quantum)
    if n == 0:
        return sign
    r = n * quantum
    if r >= Fraction(2) ** 128:
        return sign | 0x7F80
    # encode r = n * 2^(e-7), n <= 256
    ee = floor_log2(r)
    if ee < -126:  # subnormal: fraction field = r / 2^-133
        return sign | int(r / Fraction(2) ** -133)
    frac = (r / Fraction(2) ** ee - 1) * 128
    assert frac.denominator == 1
    return sign | ((ee + 127) << 7) | int(frac)


def f32_value(x: float) -> Fraction:
    return Fraction(x)


E2M1_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def e2m1_bits_value(code: int) -> Fraction:
    """E2M1 from its bit fields: sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent 0
    is subnormal (value = mantissa * 1/2)."""
    s = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2)
    else:
        mag = (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return s * mag


def ue4m3_bits_value(b: int) -> Fraction:
    """Unsigned E4M3 from its bit fields: 4-bit exponent (bias 7), 3-bit mantissa;
    exponent 0 is subnormal (value = m/8 * 2^-6)."""
    e = (b >> 3) & 15
    m = b & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(2) ** -6
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
