"""Test helpers: exact rational rounding and ULP distances.

Independent of both the oracle and the HIP path: these functions restate the
IEEE-754 rounding rule on exact rationals (``fractions.Fraction``), so the
oracle's binary32 / BF16 mechanics can be checked against arithmetic that
has no rounding of its own.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np

F32 = dict(p=24, emin=-126, emax=127)
BF16 = dict(p=8, emin=-126, emax=127)


def exact(x) -> Fraction:
    """The exact rational value of a finite float (Python float or numpy scalar)."""
    return Fraction(float(x))


def round_rne(q: Fraction, p: int, emin: int, emax: int) -> Fraction:
    """Rounds q to the nearest value with a p-bit significand (ties to even),
    with gradual underflow below 2^emin; returns +-inf as a float on overflow."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * r


def f32(q: Fraction) -> float:
    """Exact rational -> binary32 value (as a Python float), RNE."""
    r = round_rne(q, **F32)
    return float(r)


def bf16_bits_of(q: Fraction) -> int:
    """Exact rational -> BF16 bit pattern, RNE (a zero result is +0 unless q is
    a signed zero, which rationals cannot express)."""
    r = round_rne(q, **BF16)
    f = float(r)
    return struct.unpack("<I", struct.pack("<f", f))[0] >> 16


def bf16_value(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_ulp_distance(a, b) -> np.ndarray:
    """|steps| between BF16 bit patterns on the ordered number line (+0 == -0)."""
    def key(x):
        x = np.asarray(x, dtype=np.int64)
        return np.where(x < 0x8000, 0x8000 + x, 0x8000 - (x - 0x8000))
    return np.abs(key(a) - key(b))


def f32_ulp_distance(a, b) -> np.ndarray:
    def key(x):
        x = np.asarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
        return np.where(x >= 0, x, -(x & 0x7FFFFFFF))
    return np.abs(key(a) - key(b))
