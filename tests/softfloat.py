"""Exact-rational IEEE-754 arithmetic for pinning the oracle.

Every value is a Python ``Fraction`` (or +-inf / nan as floats).  Each operation
computes the exact result and rounds it once to the target format (nearest,
ties to even, gradual underflow, overflow to infinity).  Used only by tests to
re-evaluate the oracle's step on tiny shards with no help from the C compiler,
the FPU or numpy, so that contraction, excess precision, a flushed subnormal
or a wrong rounding in the oracle shows up as a mismatch.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

INF = float("inf")

# (precision p incl. hidden bit, emin, emax)
F32 = (24, -126, 127)
F64 = (53, -1022, 1023)
BF16 = (8, -126, 127)


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix up
    if e >= 0:
        if a < Fraction(1 << e):
            e -= 1
    else:
        if a < Fraction(1, 1 << -e):
            e -= 1
    return e


def _pow2(e: int) -> Fraction:
    return Fraction(1 << e) if e >= 0 else Fraction(1, 1 << -e)


def rnd(x, fmt=F32):
    """Round an exact value to the format (returns Fraction, +-inf or nan)."""
    if isinstance(x, float):
        if math.isnan(x) or math.isinf(x):
            return x
        x = Fraction(x)
    p, emin, emax = fmt
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = -x if x < 0 else x
    e = max(_floor_log2(a), emin)
    q = e - p + 1                    # exponent of the last significand bit
    scaled = a / _pow2(q)
    n = scaled.numerator // scaled.denominator
    r = scaled - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    res = n * _pow2(q)
    if res >= _pow2(emax + 1):
        return s * INF
    return s * res


def _special(*xs):
    return any(isinstance(x, float) for x in xs)


def add(a, b, fmt=F32):
    if _special(a, b):
        return rnd(float(a) + float(b), fmt)
    return rnd(a + b, fmt)


def sub(a, b, fmt=F32):
    if _special(a, b):
        return rnd(float(a) - float(b), fmt)
    return rnd(a - b, fmt)


def mul(a, b, fmt=F32):
    if _special(a, b):
        return rnd(float(a) * float(b), fmt)
    return rnd(a * b, fmt)


def div(a, b, fmt=F32):
    if _special(a, b) or b == 0:
        fa, fb = float(a), float(b)
        if fb == 0:
            return float("nan") if fa == 0 else math.copysign(INF, fa)
        return rnd(fa / fb, fmt)
    return rnd(a / b, fmt)


def sqrt(a, fmt=F32):
    """Correctly rounded square root of a >= 0."""
    if isinstance(a, float):
        return math.sqrt(a) if a >= 0 else float("nan")
    if a < 0:
        return float("nan")
    if a == 0:
        return Fraction(0)
    p, emin, emax = fmt
    k = _floor_log2(a)
    e = k // 2                        # floor(log2(sqrt(a)))
    q = e - p + 1
    y = a / _pow2(2 * q)              # sqrt(a) / 2^q = sqrt(y)
    n = math.isqrt(y.numerator // y.denominator)
    half = Fraction(2 * n + 1, 2)
    if y > half * half or (y == half * half and n % 2 == 1):
        n += 1
    return n * _pow2(q)


# ---------------------------------------------------------------- conversions
def from_f32(x) -> Fraction:
    x = float(x)
    if math.isnan(x) or math.isinf(x):
        return x
    return Fraction(x)


def from_bf16_bits(h: int):
    return from_f32(struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))[0])


def to_f32(x) -> float:
    return float(x)


def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def to_bf16_bits(x) -> int:
    """Nearest-even bf16 bit pattern of an exact binary32 value."""
    if isinstance(x, float) and math.isnan(x):
        return 0x7FC0
    r = rnd(x, BF16)
    return f32_bits(float(r)) >> 16
