"""Exact rational arithmetic with explicit IEEE rounding, for tests.

This is an independent route to the correctly rounded results the
oracle must produce: values are ``fractions.Fraction`` and every rounding
to binary32 or BF16 is done here by integer arithmetic, with no float
hardware involved.  Infinity is represented by ``math.inf`` (signed).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np

F32_MANT = 23
F32_EMIN = -126
F32_EMAX = 127
BF16_MANT = 7


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e may overshoot or undershoot by one.
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_binary(q, mant_bits: int):
    """Round a Fraction to the binary format with ``mant_bits`` fraction
    bits and binary32's exponent range, nearest with ties to even."""
    if isinstance(q, float) and math.isinf(q):
        return q
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), F32_EMIN)
    quantum = Fraction(2) ** (e - mant_bits)
    r = a / quantum
    n = r.numerator // r.denominator
    rem = r - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * quantum
    if v >= Fraction(2) ** (F32_EMAX + 1):
        return sign * math.inf
    return sign * v


def rn_f32(q):
    return _round_binary(q, F32_MANT)


def rn_bf16(q):
    return _round_binary(q, BF16_MANT)


def f32_of(x) -> Fraction:
    """Exact value of a binary32 number (finite)."""
    return Fraction(float(np.float32(x)))


def bf16_bits_to_fraction(b: int):
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    if math.isinf(f):
        return f
    return Fraction(f)


def value_to_bf16_bits(v) -> int:
    """Bits of an exactly representable BF16 value (or signed Inf)."""
    if isinstance(v, float) and math.isinf(v):
        return 0x7F80 if v > 0 else 0xFF80
    f = float(v)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert u & 0xFFFF == 0, "value is not a BF16 value"
    return u >> 16


def round_half_even_int(q: Fraction) -> int:
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", float(np.float32(x))))[0]


def from_hex_or_rational(tok: str) -> Fraction:
    """Parse '0x1p-133', '3/127', '-40.25' exactly."""
    tok = tok.strip()
    if "/" in tok:
        num, den = tok.split("/")
        return from_hex_or_rational(num) / from_hex_or_rational(den)
    if "x" in tok.lower():
        return Fraction(float.fromhex(tok))
    return Fraction(tok)
