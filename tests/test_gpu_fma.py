"""GPU parity for the declared fused multiply-add convention.

The pages keep multiply and add unfused (OPEN-1B paper, section 2.1 "Fused
multiply-add"); repro_gemm_fma declares the fused chain instead:
acc = fma(a, b, acc), k ascending, one rounding per step, under the same
subnormal rule.  Before any GEMM is trusted, each unit's single step is
compared with the oracle's fma on directed operand sets:
  unit 0 - VALU v_fma_f32
  unit 1 - v_mfma_f32_32x32x1_2b_f32 with the chain value as C (K = 1)
  unit 2 - v_mfma_f32_16x16x1_4b_f32, the same way
  unit 3 - v_mfma_f32_4x4x1_16b_f32, the same way
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

UNITS = [0, 1, 2, 3]


def _triples(seed, n):
    rng = np.random.default_rng(seed)

    def rnd(lo, hi):
        m = rng.uniform(1, 2, n) * rng.choice([-1, 1], n)
        return (m * 2.0 ** rng.integers(lo, hi, n)).astype(np.float32)

    sets = []
    # Random exponents, with c near -a*b for a third (cancellation).
    a, b, c = rnd(-70, 60), rnd(-70, 60), rnd(-140, 120)
    k = n // 3
    c[:k] = (-(a[:k].astype(np.float64) * b[:k]) * (1 + rng.normal(0, 1e-6, k))).astype(np.float32)
    sets.append((a, b, c))
    # Products and sums around 2^-126, c of both signs, subnormal c.
    a = (rng.uniform(1, 2, n) * 2.0 ** -63).astype(np.float32)
    b = (rng.uniform(0.5, 1, n) * 2.0 ** -63).astype(np.float32)
    c = (rng.choice([-1, 1], n) * rng.uniform(0, 2, n) * 2.0 ** -126).astype(np.float32)
    c[::5] = (rng.uniform(0, 1, c[::5].size) * 2.0 ** -126).astype(np.float32)  # includes subnormals
    sets.append((a, b, c))
    # Subnormal multiplicands.
    a = rnd(-150, -120)
    b = rnd(-10, 10)
    c = rnd(-130, -100)
    sets.append((a, b, c))
    # Exact ties after one rounding, and the double-rounding family
    # a*b + c = 1 + 2^-24 + k^2 2^-70.
    kk = rng.integers(1, 4000, n)
    a = (1 + kk * 2.0 ** -23).astype(np.float32)
    b = (-(2.0 ** -24) * (1 - kk * 2.0 ** -23)).astype(np.float32)
    c = np.full(n, 1 + 2.0 ** -23, np.float32)
    sets.append((a, b, c))
    # Signed zeros and exact cancellation.
    z = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -126, -(2.0 ** -126)], np.float32)
    g = np.array(np.meshgrid(z, z, z)).reshape(3, -1).astype(np.float32)
    sets.append((g[0], g[1], g[2]))
    return [tuple(np.ascontiguousarray(x) for x in s) for s in sets]


@pytest.mark.parametrize("unit", UNITS)
def test_single_step_matches_oracle(unit):
    for si, (a, b, c) in enumerate(_triples(100 + unit, 200_003)):
        ref = oracle.fma(a, b, c)
        got = to_host(br.repro_fp32_fma(to_dev(a), to_dev(b), to_dev(c), unit=unit))
        assert_bitwise(got, ref, f"unit {unit} set {si}")


def _product_sets(seed, n):
    """Operand pairs for the bare product: flush boundary, exact ties,
    subnormal operands against large ones, overflow, and random exponents."""
    rng = np.random.default_rng(seed)
    sign = lambda: rng.choice([-1.0, 1.0], n)
    sets = {}
    # a * b within a few ulps of 2^-126 on both sides: mantissas near 1 and
    # just below 2, at 2^-63; includes products that round up to 2^-126.
    def near(lo):
        k = rng.integers(1, 10, n)
        top = rng.random(n) < 0.5
        m = np.where(top, 2.0 - k * 2.0 ** -23, 1.0 + (k - 5) * 2.0 ** -23)
        return (m * 2.0 ** np.where(top, lo - 1, lo) * sign()).astype(np.float32)
    sets["boundary"] = (near(-63), near(-63))
    # Exact ties at 24 bits: (1 + i 2^-12)(1 + j 2^-12) with i j odd.
    i = 2 * rng.integers(0, 2000, n) + 1
    j = 2 * rng.integers(0, 2000, n) + 1
    e = rng.integers(-60, 60, n)
    sets["ties"] = (((1 + i * 2.0 ** -12) * 2.0 ** e * sign()).astype(np.float32),
                    ((1 + j * 2.0 ** -12) * 2.0 ** -e * sign()).astype(np.float32))
    # Subnormal operands times large ones (normal if the operand were not
    # read as zero), both orders.
    sub = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(-149, -127, n) * sign()).astype(np.float32)
    big = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(20, 127, n) * sign()).astype(np.float32)
    half = n // 2
    sets["subnormal"] = (np.concatenate([sub[:half], big[half:]]), np.concatenate([big[:half], sub[half:]]))
    # Overflow to infinity, and products just around the largest binary32.
    a = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(60, 127, n) * sign()).astype(np.float32)
    b = (rng.uniform(1, 2, n) * 2.0 ** rng.integers(60, 127, n) * sign()).astype(np.float32)
    m = a[::2].size  # half the pairs land within a few ulps of the largest binary32, on both sides
    a[::2] = (rng.uniform(1, 2, m) * 2.0 ** 64 * sign()[::2]).astype(np.float32)
    fmax = float(np.finfo(np.float32).max)
    b[::2] = (fmax / np.abs(a[::2].astype(np.float64)) * (1 + rng.integers(-6, 7, m) * 2.0 ** -24)
              * sign()[::2]).astype(np.float32)
    sets["overflow"] = (a, b)
    # Random exponents over the whole range.
    sets["random"] = ((rng.uniform(1, 2, n) * 2.0 ** rng.integers(-126, 64, n) * sign()).astype(np.float32),
                      (rng.uniform(1, 2, n) * 2.0 ** rng.integers(-64, 64, n) * sign()).astype(np.float32))
    z = np.array([0.0, -0.0, 1.0, -1.0, 2.0 ** -126, -(2.0 ** -126), 2.0 ** -140], np.float32)
    g = np.array(np.meshgrid(z, z)).reshape(2, -1).astype(np.float32)
    sets["zeros"] = (g[0], g[1])
    return {k: (np.ascontiguousarray(a), np.ascontiguousarray(b)) for k, (a, b) in sets.items()}


@pytest.mark.parametrize("unit", UNITS)
def test_step_with_negative_zero_is_the_product(unit):
    # With C = -0 (the identity of IEEE addition, which keeps a zero
    # product's sign) a single step is the bare product fl(a * b) under the
    # contract, bit for bit, on every unit.  The unfused GEMM's default kernel
    # takes its products from v_mfma_f32_32x32x1_2b_f32 (unit 1) this way.
    for name, (a, b) in _product_sets(300 + unit, 100_003).items():
        ref = oracle.fp32_op(oracle.OP_MUL, a, b)
        if name == "overflow":
            assert np.isinf(ref).sum() > a.size // 4 and (np.abs(ref[np.isfinite(ref)]) > 3e38).sum() > a.size // 8
        if name == "boundary":
            assert (ref == 0).any() and (np.abs(ref) == np.float32(2.0 ** -126)).any()
        c = np.full(a.size, -0.0, np.float32)
        got = to_host(br.repro_fp32_fma(to_dev(a), to_dev(b), to_dev(c), unit=unit))
        assert_bitwise(got, ref, f"unit {unit} products {name}")


@pytest.mark.parametrize("unit", [1, 2, 3])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 130, 4097])
def test_mfma_unit_ragged_groups(n, unit):
    a, b, c = (synth.generate(n, synth.NORMAL, 0x9100 + i, 1.0) for i in range(3))
    out = torch.full((n + 64,), 7.0, device="cuda")
    br.repro_fp32_fma(to_dev(a), to_dev(b), to_dev(c), unit=unit, out=out[:n])
    assert_bitwise(to_host(out[:n]), oracle.fma(a, b, c), f"n={n} unit={unit}")
    assert (to_host(out[n:]) == 7.0).all()  # nothing past the end was written


def _mat(rows, cols, tid, std=1.0):
    return synth.generate(rows * cols, synth.NORMAL, tid, std).reshape(rows, cols)


SHAPES = [(1, 1, 1), (64, 64, 64), (200, 130, 77), (129, 257, 33), (3, 700, 5), (130, 66, 16), (17, 19, 1000)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_fused_gemm_shapes_transposes_variants(M, N, K, ta, tb):
    tid = 0x9200 + M + 7 * N + 13 * K
    A = _mat(K, M, tid) if ta else _mat(M, K, tid)
    B = _mat(N, K, tid + 1, 0.5) if tb else _mat(K, N, tid + 1, 0.5)
    ref = oracle.gemm(A, B, bool(ta), bool(tb), fused=True)
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1):
        C = br.repro_gemm_fma(dA, dB, bool(ta), bool(tb), variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} ta={ta} tb={tb} fused variant={variant}")


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_fused_several_tiles_with_ragged_edges(ta, tb):
    M, N, K = 300, 400, 500  # 3 x 4 tiles, partial last tiles and a partial last k-slab of 32
    tid = 0x9800 + 2 * ta + tb
    A = _mat(K, M, tid) if ta else _mat(M, K, tid)
    B = _mat(N, K, tid + 1, 0.5) if tb else _mat(K, N, tid + 1, 0.5)
    ref = oracle.gemm(A, B, bool(ta), bool(tb), fused=True)
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1):
        C = br.repro_gemm_fma(dA, dB, bool(ta), bool(tb), variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} ta={ta} tb={tb} fused variant={variant}")


@pytest.mark.parametrize("K", [96, 77])
@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_fused_large_output_tiles_every_word(ta, tb, K):
    # 4173 x 4141 outputs (561 tiles of 256 x 128, partial in M and N): the
    # VALU variant takes its large-output kernel.  K = 96 is whole slabs for
    # both kernels (six 16-deep on the VALU, three 32-deep on the matrix
    # cores), K = 77 ends in a partial one.  Every word against the oracle's
    # fused chains, and the matrix-core variant against it.
    M, N = 4173, 4141
    tid = 0x9900 + 4 * ta + 2 * tb + (K & 1)
    A = _mat(K, M, tid) if ta else _mat(M, K, tid)
    B = _mat(N, K, tid + 1, 0.5) if tb else _mat(K, N, tid + 1, 0.5)
    ref = oracle.gemm(A, B, bool(ta), bool(tb), fused=True)
    dA, dB = to_dev(A), to_dev(B)
    C1 = br.repro_gemm_fma(dA, dB, bool(ta), bool(tb), variant=1)
    assert_bitwise(to_host(C1), ref, f"{M}x{N}x{K} ta={ta} tb={tb} fused variant=1")
    C0 = br.repro_gemm_fma(dA, dB, bool(ta), bool(tb), variant=0)
    assert torch.equal(C0.view(torch.int32), C1.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(1024, 1024, 32), (1024, 1024, 64), (4096, 4096, 16), (1024, 512, 1)])
def test_fused_slab_count_edges(M, N, K):
    # Interior tiles with one or two whole 32-deep slabs on the matrix cores,
    # one whole 16-deep slab on the VALU kernel's large-output tiles, K = 1:
    # every word against the oracle's fused chains, both variants.
    tid = 0x9A00 + K + (M >> 10)
    A = _mat(M, K, tid)
    B = _mat(K, N, tid + 1, 0.5)
    ref = oracle.gemm(A, B, fused=True)
    dA, dB = to_dev(A), to_dev(B)
    for variant in (0, 1):
        C = br.repro_gemm_fma(dA, dB, variant=variant)
        assert_bitwise(to_host(C), ref, f"{M}x{N}x{K} fused variant={variant}")


def test_fused_witness_and_difference_from_unfused():
    t = np.float32(1.0 + 2.0 ** -12)
    A = np.array([[-1.0, t]], np.float32)
    B = np.array([[1.0], [t]], np.float32)
    for variant in (0, 1):
        got = to_host(br.repro_gemm_fma(to_dev(A), to_dev(B), variant=variant))[0, 0]
        assert got == np.float32(2.0 ** -11 + 2.0 ** -24)
    # On generic data the fused and unfused chains differ somewhere.
    A = _mat(64, 256, 0x9300)
    B = _mat(256, 64, 0x9301)
    f = to_host(br.repro_gemm_fma(to_dev(A), to_dev(B)))
    u = to_host(br.repro_gemm(to_dev(A), to_dev(B)))
    assert (f.view(np.uint32) != u.view(np.uint32)).any()


def test_fused_gemm_views_and_subnormals():
    M, N, K = 70, 90, 50
    big_a = _mat(M + 3, K + 5, 0x9400)
    big_b = _mat(K + 2, N + 6, 0x9401)
    big_a[5:9, 7:20] *= np.float32(2.0 ** -66)
    big_b[3:30, 2:5] *= np.float32(2.0 ** -66)
    A = np.ascontiguousarray(big_a[1:1 + M, 3:3 + K])
    B = np.ascontiguousarray(big_b[2:2 + K, 1:1 + N])
    ref = oracle.gemm(A, B, fused=True)
    dA = to_dev(big_a)[1:1 + M, 3:3 + K]
    dB = to_dev(big_b)[2:2 + K, 1:1 + N]
    for variant in (0, 1):
        big_c = torch.zeros((M + 1, N + 9), device="cuda")
        out = big_c[1:, 3:3 + N]
        br.repro_gemm_fma(dA, dB, out=out, variant=variant)
        assert_bitwise(to_host(out), ref, f"views variant {variant}")
        rest = to_host(big_c).copy()
        rest[1:, 3:3 + N] = 0
        assert (rest == 0).all()


def test_fused_subnormal_chains_on_interior_tiles():
    # 256 x 256 x 64 with 16-byte rows: every tile of both kernels takes the
    # unchecked interior loop.  Products and chains around 2^-126: the fused
    # step rounds a * b + c once, then the result flushes if it is tiny.
    M, N, K = 256, 256, 64
    A = _mat(M, K, 0x9B00)
    B = _mat(K, N, 0x9B01)
    A[::3] *= np.float32(2.0 ** -63)
    B[:, ::2] *= np.float32(2.0 ** -63)
    A[::5, ::7] = np.float32(2.0 ** -130)
    ref = oracle.gemm(A, B, fused=True)
    assert (ref == 0).any() and (np.abs(ref[ref != 0]) < np.float32(2.0 ** -120)).any()
    for variant in (0, 1):
        C = br.repro_gemm_fma(to_dev(A), to_dev(B), variant=variant)
        assert_bitwise(to_host(C), ref, f"interior subnormal chains variant={variant}")


def test_fused_forward_workload_full_size_sampled():
    cfg = synth.GEMM
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    print(f"fused gemm workload {M}x{N}x{K}", flush=True)
    X = synth.gemm_x().reshape(M, K)
    W = synth.gemm_w().reshape(K, N)
    dX, dW = to_dev(X), to_dev(W)
    Y0 = br.repro_gemm_fma(dX, dW, variant=0)
    Y1 = br.repro_gemm_fma(dX, dW, variant=1)
    assert torch.equal(Y0.view(torch.int32), Y1.view(torch.int32))
    C = to_host(Y0)
    Bt = np.ascontiguousarray(W.T)
    rng = np.random.default_rng(8)
    for r in [0, 127, 128, M - 1] + rng.integers(0, M, 2).tolist():
        assert_bitwise(C[r], oracle.gemm(X[r:r + 1], Bt, trans_b=True, fused=True)[0], f"row {r}")
    for c in [0, 129, N - 1] + rng.integers(0, N, 1).tolist():
        assert_bitwise(C[:, c], oracle.gemm(X, Bt[c:c + 1], trans_b=True, fused=True)[:, 0], f"column {c}")


def test_fused_dw_workload_sampled():
    cfg = synth.DW
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    print(f"fused dW workload {M}x{N}x{K}", flush=True)
    X = synth.dw_x().reshape(K, M)
    dY = synth.dw_dy().reshape(K, N)
    dX, ddY = to_dev(X), to_dev(dY)
    G0 = br.repro_gemm_fma(dX, ddY, trans_a=True, variant=0)
    G1 = br.repro_gemm_fma(dX, ddY, trans_a=True, variant=1)
    assert torch.equal(G0.view(torch.int32), G1.view(torch.int32))
    C = to_host(G0)
    Aop = np.ascontiguousarray(X.T)
    Bt = np.ascontiguousarray(dY.T)
    for r in [0, M - 1, 1000]:
        assert_bitwise(C[r], oracle.gemm(Aop[r:r + 1], Bt, trans_b=True, fused=True)[0], f"row {r}")
    for c in [0, N - 1]:
        assert_bitwise(C[:, c], oracle.gemm(Aop, Bt[c:c + 1], trans_b=True, fused=True)[:, 0], f"column {c}")


def test_errors():
    lib = br.library()
    d = torch.zeros(64, device="cuda")
    p = d.data_ptr()
    assert lib.repro_gemm_fma(0, 0, 2, 2, 2, p, 2, p, 2, p, 2, 2, None) == -1  # no variant 2
    assert lib.repro_gemm_fma(0, 0, 2, 2, 2, p + 2, 2, p, 2, p, 2, 0, None) == -2
    assert lib.repro_fp32_fma(p, p, p, p, 4, 4, None) == -1  # units 0..3
    assert lib.repro_fp32_fma(p, p, p + 1, p, 4, 0, None) == -2
    assert lib.repro_fp32_fma(p, p, p, p, 0, 1, None) == 0
