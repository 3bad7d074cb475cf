"""Exact rational arithmetic with explicit IEEE rounding, for pinning the
oracle's rounding chains.

Every value is a ``fractions.Fraction``; ``rn`` rounds one to the nearest
value of a binary floating-point format (ties to the even significand),
given the format's significand width and its smallest normal exponent.  No
float operation is involved, so a result computed here does not depend on
how C, numpy or the FPU round: only on the chain of roundings the caller
writes down.
"""
from __future__ import annotations

from fractions import Fraction

# (significand bits including the implicit one, smallest normal exponent)
F64 = (53, -1022)
F32 = (24, -126)
BF16 = (8, -126)


def floor_log2(a: Fraction) -> int:
    """floor(log2 a) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^(e-1) < a < 2^(e+1) holds for this first guess; correct by one step
    if a < Fraction(2) ** e:
        e -= 1
    elif a >= Fraction(2) ** (e + 1):
        e += 1
    return e


def rn(v: Fraction, fmt=F32) -> Fraction:
    """v rounded to the nearest value of the format, ties to even
    (subnormals included; no overflow handling: callers stay in range)."""
    p, emin = fmt
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    neg = v < 0
    a = -v if neg else v
    e = max(floor_log2(a), emin)
    q = Fraction(2) ** (e - p + 1)           # the spacing of values around a
    n, rem = divmod(a, q)                    # a = n q + rem, 0 <= rem < q
    n = int(n)
    if rem * 2 > q or (rem * 2 == q and n % 2 == 1):
        n += 1
    r = n * q
    return -r if neg else r


def of_float(x) -> Fraction:
    """The exact value of a binary float (numpy or Python)."""
    return Fraction(float(x))


def bf16_value(bits: int) -> Fraction:
    """Exact value of a bf16 bit pattern (finite)."""
    import numpy as np
    f = np.array([int(bits) << 16], np.uint32).view(np.float32)[0]
    return Fraction(float(f))


def bf16_bits(v: Fraction) -> int:
    """Bit pattern of a value that is exactly a bf16 (after rn(..., BF16))."""
    import numpy as np
    f = np.float32(float(v))
    assert Fraction(float(f)) == v, "not a bf16 value"
    return int(np.array([f], np.float32).view(np.uint32)[0] >> 16)
