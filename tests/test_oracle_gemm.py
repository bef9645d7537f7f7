"""Pins for the oracle GEMM (CPU only).

Definition (OPEN-1B paper, section 2.1 "Reduction order" and "Fused
multiply-add"; section 6 item 1 names the GEMM reductions): every output
C[i][j] is one chain acc = +0, then acc <- fl(acc + fl(a_ik * b_kj)) for
k = 0, 1, ..., K-1 in ascending order.  The pins below come from exact
integer arithmetic, hand-derived order and fusion witnesses, and the
textbook error bound of recursive summation; none re-implements the chain.
"""
import itertools

import numpy as np
import pytest

import oracle


def _int_case(rng, M, N, K, trans_a, trans_b):
    A = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    B = rng.integers(-8, 9, size=(K, N)).astype(np.float32)
    exact = A.astype(np.int64) @ B.astype(np.int64)
    Aarg = np.ascontiguousarray(A.T) if trans_a else A
    Barg = np.ascontiguousarray(B.T) if trans_b else B
    return Aarg, Barg, exact


@pytest.mark.parametrize("trans_a,trans_b", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 9, 64), (64, 33, 31), (2, 70, 128)])
def test_exact_integer_products(trans_a, trans_b, M, N, K):
    # |partial sums| <= 64 * K < 2^24, so every operation is exact and the
    # result must equal the integer matrix product whatever the order.
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A, B, exact = _int_case(rng, M, N, K, trans_a, trans_b)
    C = oracle.gemm(A, B, bool(trans_a), bool(trans_b))
    assert C.shape == (M, N)
    np.testing.assert_array_equal(C.astype(np.float64), exact.astype(np.float64))  # exact in float64


def test_k_zero_writes_positive_zero():
    C = oracle.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32))
    assert C.shape == (3, 4)
    assert (C.view(np.uint32) == 0).all()


def test_positive_zero_start_value():
    # Every product is -0 (0 * -1): +0 + -0 = +0, so the output is +0, not -0.
    A = np.zeros((1, 3), np.float32)
    B = -np.ones((3, 1), np.float32)
    assert oracle.gemm(A, B).view(np.uint32)[0, 0] == 0


def test_ascending_k_order_witness():
    # Ascending: 2^24 + 1 -> 2^24 (tie to even), then - 2^24 -> 0.
    # Descending or any order pairing 1 with -2^24 first gives 1.
    A = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]], np.float32)
    B = np.ones((3, 1), np.float32)
    assert oracle.gemm(A, B)[0, 0] == 0.0
    rev = oracle.gemm(A[:, ::-1].copy(), B)
    assert rev[0, 0] == 1.0


def test_unfused_multiply_add_witness():
    # acc = -1 after k = 0; the k = 1 product (1 + 2^-12)^2 rounds to
    # 1 + 2^-11 before the add, so C = 2^-11 exactly.  A fused step would
    # give 2^-11 + 2^-24.
    t = np.float32(1.0 + 2.0 ** -12)
    A = np.array([[-1.0, t]], np.float32)
    B = np.array([[1.0], [t]], np.float32)
    assert oracle.gemm(A, B)[0, 0] == np.float32(2.0 ** -11)


def test_within_recursive_summation_error_bound():
    # Higham, "Accuracy and Stability of Numerical Algorithms", section 3.1:
    # a recursively summed dot product satisfies
    # |fl(x.y) - x.y| <= gamma_K * sum |x_k y_k|, gamma_K = K u / (1 - K u),
    # u = 2^-24.  A wrong index, a dropped term or a transposed operand breaks
    # this by orders of magnitude.
    rng = np.random.default_rng(3)
    for (M, N, K, ta, tb) in [(37, 29, 300, 0, 0), (16, 48, 1000, 1, 0), (20, 20, 257, 0, 1)]:
        A = rng.standard_normal((M, K)).astype(np.float32)
        B = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
        C = oracle.gemm(np.ascontiguousarray(A.T) if ta else A, np.ascontiguousarray(B.T) if tb else B,
                        bool(ta), bool(tb))
        exact = A.astype(np.float64) @ B.astype(np.float64)
        absum = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
        u = 2.0 ** -24
        gamma = K * u / (1 - K * u)
        err = np.abs(C.astype(np.float64) - exact)
        assert (err <= gamma * absum + 1e-30).all()
        # ...and it is not exact: the rounding really happens in binary32.
        assert (err > 0).any()


def test_order_changes_bits_on_mixed_magnitudes():
    # Non-vacuity: over all 5! orders of a K=5 chain on mixed-magnitude data
    # several distinct results occur, so a parity test on such data can tell
    # the declared order from others.  The identity order is the oracle's.
    rng = np.random.default_rng(11)
    a = (rng.standard_normal(5) * np.array([1e4, 1, 1e-3, 1e4, 1])).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    prods = a * b  # binary32 products (numpy rounds each one)
    results = set()
    ident = None
    for perm in itertools.permutations(range(5)):
        acc = np.float32(0.0)
        for k in perm:
            acc = np.float32(acc + prods[k])
        results.add(acc.tobytes())
        if perm == tuple(range(5)):
            ident = acc
    assert len(results) > 1
    C = oracle.gemm(a.reshape(1, 5), b.reshape(5, 1))
    assert C[0, 0].tobytes() == ident.tobytes()


def test_leading_dimension_and_strided_views():
    rng = np.random.default_rng(5)
    A = rng.integers(-4, 5, size=(6, 10)).astype(np.float32)
    B = rng.integers(-4, 5, size=(10, 7)).astype(np.float32)
    exact = (A.astype(np.int64) @ B.astype(np.int64))
    # A sub-block read through the raw C entry point with lda > K.
    import ctypes
    lib = oracle._load()
    C = np.zeros((4, 5), np.float32)
    sub_exact = A[1:5, 2:8].astype(np.int64) @ B[2:8, 1:6].astype(np.int64)
    Aptr = A.ctypes.data + (1 * 10 + 2) * 4
    Bptr = B.ctypes.data + (2 * 7 + 1) * 4
    rc = lib.oracle_gemm(0, 0, 4, 5, 6, ctypes.c_void_p(Aptr), 10, ctypes.c_void_p(Bptr), 7,
                         C.ctypes.data, 5)
    assert rc == 0
    np.testing.assert_array_equal(C.astype(np.int64), sub_exact)
    assert exact.shape == (6, 7)
