"""Pins for the oracle's fused multiply-add convention (CPU only).

The pages keep multiply and add unfused (OPEN-1B paper, section 2.1 "Fused
multiply-add"); the fused GEMM is a declared alternative.  Its definition:
fl(a*b + c) rounded once to binary32, round-to-nearest-even, subnormal
operands read as zeros of the same sign, and a result whose value rounded to
24 bits with an unbounded exponent lies below 2^-126 flushed to a zero of the
same sign (the contract's rule for every operation).

The pin is an exact rational evaluation of that definition in Python
(fractions.Fraction), which shares nothing with the oracle's binary64
round-to-odd construction.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

TWO = Fraction(2)
MIN_NORMAL = TWO ** -126


def _daz(x: np.float32) -> Fraction:
    x = np.float32(x)
    if x != 0 and abs(x) < np.float32(2.0 ** -126):
        return Fraction(0)
    return Fraction(float(x))


def _sign_neg(x: np.float32) -> bool:
    return bool(np.signbit(np.float32(x)))


def _round24(x: Fraction) -> Fraction:
    """Round a nonzero rational to 24 significant bits (nearest, ties to even), unbounded exponent."""
    ax = abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    if TWO ** e > ax:
        e -= 1
    elif TWO ** (e + 1) <= ax:
        e += 1
    q = ax / TWO ** (e - 23)  # in [2^23, 2^24)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * TWO ** (e - 23)
    return r if x > 0 else -r


def exact_fma(a, b, c) -> np.float32:
    fa, fb, fc = _daz(a), _daz(b), _daz(c)
    x = fa * fb + fc
    if x == 0:
        # IEEE sign of an exact zero sum: -0 only if both addends are -0
        # (the product's sign is the xor of the operand signs).
        pneg = _sign_neg(a) != _sign_neg(b)
        cneg = _sign_neg(c) if fc == 0 else fc < 0
        prod_zero = fa * fb == 0
        if prod_zero and fc == 0:
            return np.float32(-0.0) if (pneg and cneg) else np.float32(0.0)
        return np.float32(0.0)
    r = _round24(x)
    if abs(r) < MIN_NORMAL:
        return np.float32(-0.0) if x < 0 else np.float32(0.0)
    return np.float32(float(r))


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


def _check(a, b, c):
    a, b, c = (np.asarray(v, np.float32) for v in (a, b, c))
    got = oracle.fma(a, b, c)
    want = np.array([exact_fma(x, y, z) for x, y, z in zip(a, b, c)], np.float32)
    bad = np.nonzero(_bits(got) != _bits(want))[0]
    assert bad.size == 0, [(a[i], b[i], c[i], got[i], want[i]) for i in bad[:5]]


def test_random_across_exponents():
    rng = np.random.default_rng(1)
    n = 4000
    def rnd():
        m = rng.uniform(1, 2, n) * rng.choice([-1, 1], n)
        return (m * 2.0 ** rng.integers(-70, 60, n)).astype(np.float32)
    a, b = rnd(), rnd()
    # c near -a*b half of the time: heavy cancellation.
    c = np.where(rng.random(n) < 0.5, -(a.astype(np.float64) * b) * (1 + rng.normal(0, 1e-6, n)), rnd()).astype(np.float32)
    _check(a, b, c)


def test_results_near_the_flush_boundary():
    rng = np.random.default_rng(2)
    n = 4000
    a = (rng.uniform(1, 2, n) * 2.0 ** -63).astype(np.float32)
    b = (rng.uniform(0.5, 1, n) * 2.0 ** -63).astype(np.float32)
    # a*b lies in [2^-127, 2^-124); c moves the sum across 2^-126 both ways.
    c = (rng.choice([-1, 1], n) * rng.uniform(0, 2, n) * 2.0 ** -126).astype(np.float32)
    c[: n // 4] = 0.0
    _check(a, b, c)
    got = oracle.fma(a, b, c)
    small = (np.abs(got) > 0) & (np.abs(got) < np.float32(2.0 ** -125))
    assert (got == 0).any() and small.any()


def test_flush_after_rounding_to_24_bits():
    # a*b = 2^-126 * (1 - 2^-24) exactly: 24 significant bits, below 2^-126
    # after rounding -> flushed to zero.
    a = np.float32(1 - 2.0 ** -24)
    b = np.float32(2.0 ** -126)
    assert oracle.fma([a], [b], [np.float32(0)])[0] == 0
    assert oracle.fma([a], [b], [np.float32(-0.0)])[0] == 0
    # a*b = 2^-126 * (1 - 2^-26) = 2^-126 (1 - 2^-13)(1 + 2^-13): below 2^-126
    # before rounding, exactly 2^-126 after rounding to 24 bits -> kept.
    a2 = np.float32(1 - 2.0 ** -13)
    b2 = np.float32(2.0 ** -126 * (1 + 2.0 ** -13))
    assert oracle.fma([a2], [b2], [np.float32(0)])[0] == np.float32(2.0 ** -126)
    # (2^-125 + 2^-148) - (2^-126 + 2^-148) = 2^-126 exactly.
    a3, b3 = np.float32(1 + 2.0 ** -23), np.float32(2.0 ** -125)
    c3 = np.float32(-(2.0 ** -126) * (1 + 2.0 ** -22))
    assert oracle.fma([a3], [b3], [c3])[0] == np.float32(2.0 ** -126)
    _check([a, a2, a3], [b, b2, b3], [np.float32(0), np.float32(0), c3])


def test_subnormal_addend_reads_as_zero():
    c = np.float32(2.0 ** -130)
    a, b = np.float32(2.0 ** -60), np.float32(2.0 ** -60)
    got = oracle.fma([a], [b], [c])[0]
    assert got == np.float32(2.0 ** -120)  # not 2^-120 * (1 + 2^-10)
    _check([a, np.float32(2.0 ** -140)], [b, np.float32(3.0)], [c, np.float32(-1.0)])


@pytest.mark.parametrize("k", [1, 2, 3, 7, 100, 255])
def test_no_double_rounding(k):
    # a*b + c = 1 + 2^-24 + k^2 * 2^-70: just above the halfway point between
    # 1 and 1 + 2^-23, so the one rounding goes up.  Rounding to binary64
    # first (nearest) lands exactly on the halfway point and a second
    # rounding to 24 bits goes down to the even 1.
    a = np.float32(1 + k * 2.0 ** -23)
    b = np.float32(-(2.0 ** -24) * (1 - k * 2.0 ** -23))
    c = np.float32(1 + 2.0 ** -23)
    assert oracle.fma([a], [b], [c])[0] == np.float32(1 + 2.0 ** -23)
    naive = np.float32(float(a) * float(b) + float(c))
    assert naive == np.float32(1.0)
    _check([a], [b], [c])


def test_signed_zeros():
    z, nz, one = np.float32(0), np.float32(-0.0), np.float32(1)
    cases = [(z, one, nz), (nz, one, nz), (nz, one, z), (one, one, np.float32(-1)), (nz, nz, nz)]
    a, b, c = zip(*cases)
    _check(a, b, c)


def test_fused_witness():
    # (1 + 2^-12)^2 - 1: the fused result keeps the 2^-24 term, the unfused drops it.
    a = np.float32(1 + 2.0 ** -12)
    assert oracle.fma([a], [a], [np.float32(-1)])[0] == np.float32(2.0 ** -11 + 2.0 ** -24)
    A = np.array([[a, np.float32(-1)]], np.float32)
    B = np.array([[a], [np.float32(1)]], np.float32)
    # Chain: acc = fma(a, a, +0) = fl(a*a) = 1 + 2^-11 (rounded), then
    # fma(-1, 1, acc) = 2^-11 exactly.  Starting from +0 the first step is a product.
    assert oracle.gemm(A, B, fused=True)[0, 0] == np.float32(2.0 ** -11)
    A2 = np.array([[np.float32(-1), a]], np.float32)
    B2 = np.array([[np.float32(1)], [a]], np.float32)
    assert oracle.gemm(A2, B2, fused=True)[0, 0] == np.float32(2.0 ** -11 + 2.0 ** -24)
    assert oracle.gemm(A2, B2)[0, 0] == np.float32(2.0 ** -11)


def _exact_chain(A, B):
    M, K = A.shape
    N = B.shape[1]
    C = np.empty((M, N), np.float32)
    for i in range(M):
        for j in range(N):
            acc = np.float32(0)
            for k in range(K):
                acc = exact_fma(A[i, k], B[k, j], acc)
            C[i, j] = acc
    return C


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_gemm_chain_matches_exact_fma_chain(ta, tb):
    rng = np.random.default_rng(10 + 2 * ta + tb)
    M, N, K = 3, 4, 19
    A = (rng.standard_normal((M, K)) * 2.0 ** rng.integers(-8, 8, (M, K))).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    want = _exact_chain(A, B)
    Ai = np.ascontiguousarray(A.T) if ta else A
    Bi = np.ascontiguousarray(B.T) if tb else B
    got = oracle.gemm(Ai, Bi, trans_a=bool(ta), trans_b=bool(tb), fused=True)
    np.testing.assert_array_equal(_bits(got), _bits(want))


def test_gemm_fused_equals_unfused_when_every_step_is_exact():
    rng = np.random.default_rng(4)
    A = rng.integers(-50, 51, (9, 33)).astype(np.float32)
    B = rng.integers(-50, 51, (33, 7)).astype(np.float32)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    np.testing.assert_array_equal(oracle.gemm(A, B, fused=True), exact)
    np.testing.assert_array_equal(oracle.gemm(A, B), exact)
