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
    for variant in (0, 1, 2, 3, 4):
        C = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} ta={ta} tb={tb} variant={variant}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_many_tiles_with_ragged_edges(ta, tb):
    # 1000 x 1500 x 700: 8 x 12 tiles of 128 with partial last tiles in M and
    # N, and a partial last k-slab (21 of 32 plus 28; 43 of 16 plus 12), for every variant.
    M, N, K = 1000, 1500, 700
    A, B = _stored(M, N, K, ta, tb, 0x8800 + 2 * ta + tb)
    ref = oracle.gemm(A, B, bool(ta), bool(tb))
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1, 2, 3, 4):
        C = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} ta={ta} tb={tb} variant={variant}")


@pytest.mark.parametrize("K", [96, 77])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_large_output_tiles_every_word(ta, tb, K):
    # 4173 x 4141 outputs: 17 x 33 = 561 tiles of 256 x 128, enough for the
    # VALU variant 4 to take its large-output kernel, with partial tiles in
    # M and N.  K = 96 is three whole 32-deep slabs of the default kernel and
    # six 16-deep ones of variant 4 (interior tiles take the unchecked
    # loads), K = 77 ends in a partial slab (every tile checked).
    # Every output word of the default (matrix-core products) and of
    # variant 4 against the oracle, and variant 1's 128 x 128 kernel against
    # them.
    M, N = 4173, 4141
    A, B = _stored(M, N, K, ta, tb, 0x8900 + 4 * ta + 2 * tb + (K & 1))
    ref = oracle.gemm(A, B, bool(ta), bool(tb))
    dA, dB = to_dev(A), to_dev(B)
    C0 = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=0)
    assert_bitwise(to_host(C0), ref, f"{M}x{N}x{K} ta={ta} tb={tb} variant=0")
    C4 = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=4)
    assert_bitwise(to_host(C4), ref, f"{M}x{N}x{K} ta={ta} tb={tb} variant=4")
    C1 = br.repro_gemm(dA, dB, bool(ta), bool(tb), variant=1)
    assert torch.equal(C0.view(torch.int32), C1.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 16), (4096, 4096, 8), (4096, 4096, 1), (512, 640, 32),
                                   (1024, 1024, 64), (1024, 1024, 48)])
def test_slab_count_edges(M, N, K):
    # Interior tiles with one or two whole slabs (K = 16 on the VALU kernel's
    # 256 x 128 tiles, K = 32 and 64 on the 128 x 128 ones, 32-deep), a whole
    # slab and a partial one (K = 48), a single partial slab (K = 8 or 16)
    # and K = 1: every output word against the oracle, variants 0, 1 and 4.
    A, B = _stored(M, N, K, 0, 0, 0x8A00 + K + (M & 7))
    ref = oracle.gemm(A, B)
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1, 4):
        C = br.repro_gemm(dA, dB, variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} variant={variant}")


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


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
def test_subnormal_operands_and_products(variant):
    # Subnormal inputs read as zero; products below 2^-126 flush; the chain's
    # exact subnormal sums flush.  Compared with the oracle's rule, for every
    # variant (variants 0 and 3 form the products on the matrix cores).
    # 256 x 256 x 64 takes the unchecked interior loop, 32 x 32 x 40 the
    # checked one.
    rng = np.random.default_rng(5)
    for M, N, K in ((32, 32, 40), (256, 256, 64)):
        A = (rng.standard_normal((M, K)) * 2.0 ** -63).astype(np.float32)
        B = (rng.standard_normal((K, N)) * 2.0 ** -63).astype(np.float32)
        A[::3, ::2] = np.float32(2.0 ** -130)
        ref = oracle.gemm(A, B)
        assert_bitwise(to_host(br.repro_gemm(to_dev(A), to_dev(B), variant=variant)), ref,
                       f"{M}x{N}x{K} subnormal products variant={variant}")


def _boundary_operands(rng, rows, cols):
    """Operands whose pairwise products sit on the flush boundary: mantissas
    within a few ulps of 1 (and of 2) times 2^-63, both signs, so that a * b
    lands within ulps of 2^-126 on either side; plus exact zeros of both signs,
    subnormals and the smallest normal."""
    k = rng.integers(-4, 5, (rows, cols))
    top = rng.random((rows, cols)) < 0.5
    mant = np.where(top, 2.0 - (k + 5) * 2.0 ** -23, 1.0 + k * 2.0 ** -23)
    x = mant * 2.0 ** np.where(top, -64, -63) * rng.choice([-1.0, 1.0], (rows, cols))
    special = np.array([0.0, -0.0, 2.0 ** -149, -(2.0 ** -140), 2.0 ** -126, -(2.0 ** -126)])
    mask = rng.random((rows, cols)) < 0.15
    x = np.where(mask, special[rng.integers(0, special.size, (rows, cols))], x)
    return x.astype(np.float32)


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
def test_directed_flush_boundary_products(variant):
    # Every product a * b is within a few ulps of +-2^-126 (or a zero or
    # subnormal operand), so each step's product is decided by the flush rule:
    # tiny after rounding -> signed zero, otherwise the rounded product.  The
    # chain then adds values of a few times 2^-126, whose exact sums are normal
    # or flush.  One GEMM per variant against the oracle, plus the K = 1 case
    # where every output is a single product; 256 x 256 x 64 has 16-byte rows
    # and whole slabs, so its tiles take the unchecked interior loop.
    rng = np.random.default_rng(11)
    for M, N, K in ((64, 64, 1), (96, 80, 37), (130, 129, 64), (256, 256, 64)):
        A = _boundary_operands(rng, M, K)
        B = _boundary_operands(rng, K, N)
        ref = oracle.gemm(A, B)
        got = to_host(br.repro_gemm(to_dev(A), to_dev(B), variant=variant))
        assert_bitwise(got, ref, f"{M}x{N}x{K} boundary variant={variant}")
        # The set really straddles the boundary: some products flush, some survive.
        p = oracle.fp32_op(oracle.OP_MUL, np.repeat(A[:, :1], N, 1).reshape(-1), np.tile(B[0], M))
        assert (p == 0).any() and (np.abs(p) >= np.float32(2.0 ** -126)).any()


@pytest.mark.parametrize("variant", [0, 1, 2, 3, 4])
def test_overflowing_products(variant):
    # A product beyond the largest binary32 rounds to infinity of its sign and
    # stays there along the chain; the other outputs stay finite.  256 x 256
    # x 64 takes the interior loop of every kernel.
    for M, N, K in ((70, 66, 33), (256, 256, 64)):
        _overflow_case(variant, M, N, K)


def _overflow_case(variant, M, N, K):
    rng = np.random.default_rng(12)
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    A[5, 7] = np.float32(2.0 ** 100)
    B[7, :] = (np.where(np.arange(N) % 2 == 0, 1.0, -1.0) * 2.0 ** 60).astype(np.float32)
    A[9, 3] = np.float32(-(2.0 ** 127))
    B[3, ::3] = np.float32(4.0)  # -2^127 * 4 = -2^129: beyond the largest binary32
    ref = oracle.gemm(A, B)
    assert np.isposinf(ref[5, 0]) and np.isneginf(ref[5, 1]) and np.isneginf(ref[9, 0])
    assert np.isnan(ref).sum() == 0
    got = to_host(br.repro_gemm(to_dev(A), to_dev(B), variant=variant))
    assert_bitwise(got, ref, f"overflow variant={variant}")


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


def _repeat_digests(run, out, times=10):
    """State hashes (computed on the GPU) of `out` after each of `times` runs."""
    ws = br.hash_workspace(out.numel(), out.device)
    digests = []
    for _ in range(times):
        out.fill_(7.0)
        run()
        digests.append(br.repro_state_hash(out.reshape(-1), ws))
    return digests


def test_forward_workload_full_size_sampled():
    # Y[8192 x 8192] = X[8192 x 2048] W[2048 x 8192], K = 2048.  Full rows and
    # columns at tile edges and at random positions; ten runs give one digest
    # of the whole output.
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
    first = br.repro_state_hash(Y.reshape(-1))
    digests = _repeat_digests(lambda: br.repro_gemm(dX, dW, out=Y), Y)
    assert digests == [first] * 10
    assert np.array_equal(to_host(Y).view(np.uint32), C.view(np.uint32))
    # The VALU kernel (variant 4, large-output tiles) gives the same bits.
    assert _repeat_digests(lambda: br.repro_gemm(dX, dW, out=Y, variant=4), Y, times=2) == [first] * 2


def test_weight_gradient_workload_full_size_sampled():
    # dW[2048 x 8192] = X^T dY with X[16384 x 2048], dY[16384 x 8192]: one
    # 16,384-long ascending chain per output; heavy-tailed t(3) data.  Ten
    # runs give one digest of the whole output.
    cfg = synth.DW
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    print(f"dW workload {M}x{N}x{K}", flush=True)
    X = synth.dw_x().reshape(K, M)
    dY = synth.dw_dy().reshape(K, N)
    dX, ddY = to_dev(X), to_dev(dY)
    out = br.repro_gemm(dX, ddY, trans_a=True)
    C = to_host(out)
    rng = np.random.default_rng(4)
    rows = [0, 128, M - 1] + rng.integers(0, M, 1).tolist()
    cols = [0, 255, N - 1] + rng.integers(0, N, 1).tolist()
    _sampled_check(C, X, dY, True, False, rows, cols, "dW workload")
    first = br.repro_state_hash(out.reshape(-1))
    digests = _repeat_digests(lambda: br.repro_gemm(dX, ddY, trans_a=True, out=out), out)
    assert digests == [first] * 10
    assert np.array_equal(to_host(out).view(np.uint32), C.view(np.uint32))
    assert _repeat_digests(lambda: br.repro_gemm(dX, ddY, trans_a=True, out=out, variant=4), out,
                           times=2) == [first] * 2


def test_errors():
    lib = br.library()
    d = torch.zeros(64, device="cuda")
    p = d.data_ptr()
    assert lib.repro_gemm(0, 0, 2, 2, 2, p, 1, p, 2, p, 2, None) == -1  # lda < K
    assert lib.repro_gemm(0, 0, 2, 2, 2, p + 2, 2, p, 2, p, 2, None) == -2  # misaligned A
    assert lib.repro_gemm(2, 0, 2, 2, 2, p, 2, p, 2, p, 2, None) == -1  # bad flag
    assert lib.repro_gemm(0, 0, -1, 2, 2, p, 2, p, 2, p, 2, None) == -1
