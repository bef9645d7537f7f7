"""Pins for the oracle's binary32 contract (CPU only).

OPEN-1B paper, section 2.1 ("Fused multiply-add", "Subnormals") and Table 1:
one unfused convention, and subnormals flushed to zero everywhere, with the
processor path turning on its FTZ mode (a subnormal result becomes zero) and
DAZ mode (a subnormal input reads as zero).  The reading taken is the x86
definition of those modes: round to nearest even; a subnormal operand reads
as a zero of the same sign; a result is replaced by a zero of the same sign
when it is tiny, i.e. when rounded to 24 significant bits with an unbounded
exponent it lies below 2^-126.  Every expected value here is derived by hand
from that rule.
"""
import numpy as np

import oracle
from oracle import OP_ADD, OP_DIV, OP_MUL, OP_SQRT, OP_SUB

MIN_NORMAL = np.float32(2.0 ** -126)


def f(x):
    return np.float32(x)


def bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))


def one(op, a, b=0.0):
    return oracle.fp32_op(op, np.array([a], np.float32), np.array([b], np.float32))[0]


def test_subnormal_operands_read_as_signed_zero():
    sub = f(2.0 ** -130)
    assert bits(one(OP_ADD, sub, 0.0)) == 0  # DAZ: 2^-130 + 0 -> +0
    assert bits(one(OP_ADD, -sub, -0.0)) == 0x80000000  # -0 + -0 = -0
    assert one(OP_ADD, sub, 1.0) == 1.0
    # 1 * subnormal: the operand is zero, so the product is a signed zero.
    assert bits(one(OP_MUL, 1.0, -sub)) == 0x80000000
    assert bits(one(OP_SQRT, sub)) == 0
    assert bits(one(OP_SQRT, -0.0)) == 0x80000000


def test_subnormal_results_flush_with_sign():
    # 2^-63 * 2^-64 = 2^-127 exactly: subnormal, flushed.
    assert bits(one(OP_MUL, 2.0 ** -63, 2.0 ** -64)) == 0
    assert bits(one(OP_MUL, -(2.0 ** -63), 2.0 ** -64)) == 0x80000000
    # 1.5*2^-126 - 2^-126 = 2^-127 exactly: subnormal, flushed to +0.
    assert bits(one(OP_SUB, 1.5 * 2.0 ** -126, 2.0 ** -126)) == 0
    assert bits(one(OP_ADD, 2.0 ** -126, -1.5 * 2.0 ** -126)) == 0x80000000
    assert bits(one(OP_DIV, 2.0 ** -126, 2.0)) == 0
    # The smallest normal stays.
    assert one(OP_MUL, 2.0 ** -63, 2.0 ** -63) == MIN_NORMAL
    assert one(OP_DIV, 2.0 ** -125, 2.0) == MIN_NORMAL


def test_tininess_is_decided_after_rounding_with_unbounded_exponent():
    # (1 - 2^-24) * 2^-126 = 2^-126 - 2^-150 = 2^-127 * (2 - 2^-23): exactly 24
    # significant bits, so rounding with an unbounded exponent leaves it below
    # 2^-126: tiny, flushed.  (Rounding onto the subnormal grid first would
    # give the tie 0x007FFFFF / 0x00800000 and keep 2^-126.)
    a = np.uint32(0x3F7FFFFF).view(np.float32)
    assert float(a) == 1.0 - 2.0 ** -24
    assert bits(one(OP_MUL, a, 2.0 ** -126)) == 0
    assert bits(one(OP_MUL, -a, 2.0 ** -126)) == 0x80000000
    # ((1 - 2^-13) 2^-63) * ((1 + 2^-13) 2^-63) = 2^-126 (1 - 2^-26): rounded
    # to 24 bits it is 2^-126 itself, so it is not tiny and stays.  (Deciding
    # on the exact value before rounding would flush it.)
    x = np.float32((1 - 2.0 ** -13) * 2.0 ** -63)
    y = np.float32((1 + 2.0 ** -13) * 2.0 ** -63)
    assert bits(one(OP_MUL, x, y)) == 0x00800000
    # (1 - 2^-23) * 2^-126 = 2^-126 - 2^-149: exactly subnormal, flushed.
    a2 = np.uint32(0x3F7FFFFE).view(np.float32)
    assert bits(one(OP_MUL, a2, 2.0 ** -126)) == 0
    # Quotient (2^-125 - 2^-149) / 2 = 2^-126 - 2^-150 exactly: tiny, flushed.
    q = np.uint32(0x00FFFFFF).view(np.float32)
    assert bits(one(OP_DIV, q, 2.0)) == 0


def test_unfused_multiply_then_add():
    # (1 + 2^-12)^2 = 1 + 2^-11 + 2^-24: the product rounds (tie to even) to
    # 1 + 2^-11 before the add, so -1 + that is exactly 2^-11.  A fused
    # multiply-add would keep the 2^-24 term.
    a = f(1.0 + 2.0 ** -12)
    p = one(OP_MUL, a, a)
    assert p == f(1.0 + 2.0 ** -11)
    assert one(OP_ADD, -1.0, p) == f(2.0 ** -11)


def test_round_to_nearest_even_on_ties():
    # 2^24 + 1 is a tie between 2^24 and 2^24 + 2; even mantissa is 2^24.
    assert one(OP_ADD, 2.0 ** 24, 1.0) == f(2.0 ** 24)
    # 2^24 + 3 is a tie between 2^24 + 2 and 2^24 + 4; even is 2^24 + 4.
    assert one(OP_ADD, 2.0 ** 24 + 2, 1.0) == f(2.0 ** 24 + 4)


def test_division_and_sqrt_are_correctly_rounded():
    # Against the host's IEEE routines on normal inputs whose results stay
    # normal (numpy float32 division and sqrt are the SSE instructions).
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    b = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    np.testing.assert_array_equal(oracle.fp32_op(OP_DIV, a, b), a / b)
    np.testing.assert_array_equal(oracle.fp32_op(OP_SQRT, np.abs(a)), np.sqrt(np.abs(a)))
    # 1/3 in binary32 is 0x3EAAAAAB (0.333333343...).
    assert bits(one(OP_DIV, 1.0, 3.0)) == 0x3EAAAAAB
    assert one(OP_SQRT, 4.0) == 2.0
    assert one(OP_SQRT, 2.0) == f(np.sqrt(np.float64(2.0)))
