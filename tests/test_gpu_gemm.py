"""GPU parity: repro_gemm against the oracle GEMM, word for word.

OPEN-1B paper, section 2.1 ("Reduction order", "Fused multiply-add") and
section 6 item 1: each output is one ascending-k chain of unfused
multiply-then-add steps.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu


def _mat(rows, cols, tid, std=1.0):
    return synth.generate(rows * cols, synth.NORMAL, tid, std).reshape(rows, cols)


def _stored(M, N, K, ta, tb, tid):
    """Stored A and B (transposed storage when ta / tb) and their oracle product."""
    A = _mat(K, M, tid) if ta else _mat(M, K, tid)
    B = _mat(N, K, tid + 1, 0.5) if tb else _mat(K, N, tid + 1, 0.5)
    return A, B


SHAPES = [(1, 1, 1), (64, 64, 64), (200, 130, 77), (129, 257, 33), (3, 700, 5), (256, 256, 300), (130, 66, 16),
          (17, 19, 1000)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_shapes_transposes_variants(M, N, K, ta, tb):
    A, B = _stored(M, N, K, ta, tb, 0x8000 + M + 7 * N + 13 * K)
    ref = oracle.gemm(A, B, bool(ta), bool(tb))
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1, 2, 3):
        C = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} ta={ta} tb={tb} variant={variant}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_many_tiles_with_ragged_edges(ta, tb):
    # 1000 x 1500 x 700: 8 x 12 tiles of 128 with partial last tiles in M and
    # N, and 43 full k-slabs of 16 plus a partial one, for every variant.
    M, N, K = 1000, 1500, 700
    A, B = _stored(M, N, K, ta, tb, 0x8800 + 2 * ta + tb)
    ref = oracle.gemm(A, B, bool(ta), bool(tb))
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1, 2, 3):
        C = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} ta={ta} tb={tb} variant={variant}")


def test_tiny_workload():
    a, b = synth.tiny_gemm_inputs()
    C = br.repro_gemm(to_dev(a), to_dev(b))
    assert_bitwise(to_host(C), oracle.gemm(a, b), "tiny gemm")


def test_k_zero_and_empty():
    A = torch.zeros((5, 0), device="cuda")
    B = torch.zeros((0, 7), device="cuda")
    C = torch.full((5, 7), 3.0, device="cuda")
    br.repro_gemm(A, B, out=C)
    assert (to_host(C).view(np.uint32) == 0).all()  # +0, not -0
    br.repro_gemm(torch.zeros((0, 3), device="cuda"), torch.zeros((3, 4), device="cuda"))


def test_order_and_fusion_witnesses():
    # Ascending k: [2^24, 1, -2^24] . [1, 1, 1] = 0 (not 1).
    A = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24)]] * 3, np.float32)
    B = np.ones((3, 5), np.float32)
    assert (to_host(br.repro_gemm(to_dev(A), to_dev(B))) == 0).all()
    # Unfused: -1 + (1 + 2^-12)^2 = 2^-11 exactly (a fused step keeps 2^-24 more).
    t = np.float32(1.0 + 2.0 ** -12)
    A = np.array([[-1.0, t]], np.float32)
    B = np.array([[1.0], [t]], np.float32)
    assert to_host(br.repro_gemm(to_dev(A), to_dev(B)))[0, 0] == np.float32(2.0 ** -11)


def test_leading_dimensions_and_unaligned_views():
    M, N, K = 70, 90, 50
    big_a = _mat(M + 3, K + 5, 0x8100)
    big_b = _mat(K + 2, N + 6, 0x8101)
    A = big_a[1:1 + M, 3:3 + K]
    B = big_b[2:2 + K, 1:1 + N]
    ref = oracle.gemm(np.ascontiguousarray(A), np.ascontiguousarray(B))
    dA = to_dev(big_a)[1:1 + M, 3:3 + K]  # lda = K + 5, base 4-byte aligned only
    dB = to_dev(big_b)[2:2 + K, 1:1 + N]
    big_c = torch.zeros((M + 1, N + 9), device="cuda")
    out = big_c[1:, 3:3 + N]  # ldc = N + 9
    br.repro_gemm(dA, dB, out=out)
    assert_bitwise(to_host(out), ref, "strided views")
    # Nothing outside the output view was touched.
    rest = to_host(big_c).copy()
    rest[1:, 3:3 + N] = 0
    assert (rest == 0).all()


def test_subnormal_operands_and_products():
    # Subnormal inputs read as zero; products below 2^-126 flush; the chain's
    # exact subnormal sums flush.  Compared with the oracle's rule.
    rng = np.random.default_rng(5)
    M, N, K = 32, 32, 40
    A = (rng.standard_normal((M, K)) * 2.0 ** -63).astype(np.float32)
    B = (rng.standard_normal((K, N)) * 2.0 ** -63).astype(np.float32)
    A[::3, ::2] = np.float32(2.0 ** -130)
    ref = oracle.gemm(A, B)
    assert_bitwise(to_host(br.repro_gemm(to_dev(A), to_dev(B))), ref, "subnormal products")


def _sampled_check(C, A, B, ta, tb, rows, cols, what):
    """Compare full rows and full columns of C with the oracle on the same inputs.

    Output C[i][j] depends only on row i of op(A) and column j of op(B), so an
    oracle call on those slices computes exactly the same chains.  The
    operands are handed to the oracle as op(A) and op(B)^T, both contiguous
    along k, which keeps its k loop streaming through memory."""
    Aop = np.ascontiguousarray(A.T if ta else A)
    Bt = np.ascontiguousarray(B if tb else B.T)
    for r in rows:
        ref = oracle.gemm(Aop[r:r + 1], Bt, trans_b=True)
        assert_bitwise(C[r], ref[0], f"{what} row {r}")
    for c in cols:
        ref = oracle.gemm(Aop, Bt[c:c + 1], trans_b=True)
        assert_bitwise(C[:, c], ref[:, 0], f"{what} column {c}")


def test_forward_workload_full_size_sampled():
    # Y[8192 x 8192] = X[8192 x 2048] W[2048 x 8192], K = 2048.  Full rows and
    # columns at tile edges and at random positions; ten repeats identical.
    cfg = synth.GEMM
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    print(f"gemm workload {M}x{N}x{K}", flush=True)
    X = synth.gemm_x().reshape(M, K)
    W = synth.gemm_w().reshape(K, N)
    dX, dW = to_dev(X), to_dev(W)
    Y = br.repro_gemm(dX, dW)
    C = to_host(Y)
    rng = np.random.default_rng(3)
    rows = [0, 127, 128, 4095, M - 1] + rng.integers(0, M, 3).tolist()
    cols = [0, 127, 128, N - 1] + rng.integers(0, N, 2).tolist()
    _sampled_check(C, X, W, False, False, rows, cols, "gemm workload")
    first = Y.clone()
    for _ in range(3):
        again = br.repro_gemm(dX, dW)
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))


def test_weight_gradient_workload_full_size_sampled():
    # dW[2048 x 8192] = X^T dY with X[16384 x 2048], dY[16384 x 8192]: one
    # 16,384-long ascending chain per output; heavy-tailed t(3) data.
    cfg = synth.DW
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    print(f"dW workload {M}x{N}x{K}", flush=True)
    X = synth.dw_x().reshape(K, M)
    dY = synth.dw_dy().reshape(K, N)
    out = br.repro_gemm(to_dev(X), to_dev(dY), trans_a=True)
    C = to_host(out)
    rng = np.random.default_rng(4)
    rows = [0, 128, M - 1] + rng.integers(0, M, 1).tolist()
    cols = [0, 255, N - 1] + rng.integers(0, N, 1).tolist()
    _sampled_check(C, X, dY, True, False, rows, cols, "dW workload")


def test_errors():
    lib = br.library()
    d = torch.zeros(64, device="cuda")
    p = d.data_ptr()
    assert lib.repro_gemm(0, 0, 2, 2, 2, p, 1, p, 2, p, 2, None) == -1  # lda < K
    assert lib.repro_gemm(0, 0, 2, 2, 2, p + 2, 2, p, 2, p, 2, None) == -2  # misaligned A
    assert lib.repro_gemm(2, 0, 2, 2, 2, p, 2, p, 2, p, 2, None) == -1  # bad flag
    assert lib.repro_gemm(0, 0, -1, 2, 2, p, 2, p, 2, p, 2, None) == -1
