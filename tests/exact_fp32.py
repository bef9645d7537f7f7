"""Binary32 operations by exact rational arithmetic, under the contract's
subnormal rule, written from the definitions alone (test helper).

The rule (OPEN-1B paper, section 2.1 "Subnormals" and Table 1, read with the
x86 meaning of FTZ and DAZ): round to nearest, ties to even; a subnormal
operand reads as a zero of the same sign; a result whose value, rounded to 24
significant bits with an unbounded exponent, lies below 2^-126 in magnitude
becomes a zero of the same sign; a rounded magnitude of 2^128 or more is an
infinity.  Each operation computes its exact result as a Fraction (square
roots by integer square roots), then rounds once.  Nothing here uses the
host's floating-point arithmetic on the values, so it is independent of both
the oracle and the GPU library.
"""
from fractions import Fraction
from math import isqrt

import numpy as np

MIN_NORMAL = Fraction(1, 2 ** 126)
OVERFLOW = Fraction(2 ** 128)


def _bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).reshape(()).view(np.uint32))


def decode(x):
    """(sign, Fraction magnitude) of a binary32 word after DAZ; None for inf/NaN."""
    u = _bits(x)
    sign = u >> 31
    exp = (u >> 23) & 0xFF
    man = u & 0x7FFFFF
    if exp == 0xFF:
        return None
    if exp == 0:  # zero or subnormal: reads as a zero of the same sign
        return sign, Fraction(0)
    return sign, Fraction(man | 0x800000) * Fraction(2) ** (exp - 150)


def _encode(sign: int, mag: Fraction) -> np.float32:
    """The binary32 word of an already rounded magnitude (normal, zero or inf)."""
    if mag == 0:
        return np.array([sign << 31], np.uint32).view(np.float32)[0]
    if mag >= OVERFLOW:
        return np.float32(-np.inf if sign else np.inf)
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    if Fraction(2) ** e > mag:
        e -= 1
    man = mag / Fraction(2) ** (e - 23)
    assert man.denominator == 1 and 2 ** 23 <= man.numerator < 2 ** 24
    word = (sign << 31) | ((e + 127) << 23) | (man.numerator & 0x7FFFFF)
    return np.array([word], np.uint32).view(np.float32)[0]


def _round24(mag: Fraction) -> Fraction:
    """Round a positive magnitude to 24 significant bits, nearest-even, unbounded exponent."""
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    if Fraction(2) ** e > mag:
        e -= 1
    scale = Fraction(2) ** (e - 23)
    q = mag / scale
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n * scale


def finish(sign: int, exact: Fraction) -> np.float32:
    """Round the exact magnitude once and apply the flush and overflow rules."""
    if exact == 0:
        return _encode(sign, Fraction(0))
    r = _round24(exact)
    if r < MIN_NORMAL:
        return _encode(sign, Fraction(0))
    return _encode(sign, r)


def add(a, b) -> np.float32:
    da, db = decode(a), decode(b)
    va = -da[1] if da[0] else da[1]
    vb = -db[1] if db[0] else db[1]
    s = va + vb
    if s == 0:  # exact zero: -0 only when both operands are (read as) -0
        return _encode(1 if (da[0] and db[0] and da[1] == 0 and db[1] == 0) else 0, Fraction(0))
    return finish(1 if s < 0 else 0, abs(s))


def sub(a, b) -> np.float32:
    return add(a, np.array([_bits(b) ^ 0x80000000], np.uint32).view(np.float32)[0])


def mul(a, b) -> np.float32:
    da, db = decode(a), decode(b)
    return finish(da[0] ^ db[0], da[1] * db[1])


def div(a, b) -> np.float32:
    da, db = decode(a), decode(b)
    assert db[1] != 0, "finite quotients only"
    return finish(da[0] ^ db[0], da[1] / db[1])


def sqrt(a) -> np.float32:
    s, m = decode(a)
    if m == 0:
        return _encode(s, Fraction(0))
    assert s == 0, "non-negative operands only"
    # sqrt(m) = sqrt(Y) * 2^(e - 23) with Y = m * 2^(46 - 2e) in [2^46, 2^48).
    e = (m.numerator.bit_length() - m.denominator.bit_length()) // 2 + 1
    while Fraction(2) ** (2 * e) > m:
        e -= 1
    while Fraction(2) ** (2 * e + 2) <= m:
        e += 1
    Y = m * Fraction(2) ** (46 - 2 * e)
    n = isqrt(Y.numerator // Y.denominator)
    while Fraction((n + 1) ** 2) <= Y:
        n += 1
    # sqrt(Y) in [n, n + 1): round to nearest by comparing Y with (n + 1/2)^2.
    mid = Fraction(2 * n + 1, 2) ** 2
    if Y > mid or (Y == mid and n % 2 == 1):
        n += 1
    return finish(0, n * Fraction(2) ** (e - 23))
