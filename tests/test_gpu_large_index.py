"""GPU parity past 2^31 elements: 64-bit indexing in every kernel's address math.

The workloads stay below 2^31 elements per array, so these cases go beyond
them on purpose: a TreeFold over buffers of 2^31 + 4099 floats (the
vectorised body and the scalar tail both past 2^31), a GEMM whose output has
more than 2^31 elements (ragged edge tiles at the far corner), and a state
hash over more than 2^32 words (17 GB; leaf byte offsets past 2^34).  Inputs
are seeded device-side draws (torch's generator, not the library); the
compared windows are copied to the host and recomputed by the oracle.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
from parity_util import assert_bitwise, to_host

pytestmark = pytest.mark.gpu


def _randn(n, seed, std):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(n, generator=g, device="cuda") * std


def test_tree_reduce_past_two_to_the_31():
    n = (1 << 31) + 4099  # 16-byte body of (2^31 + 4096) / 4 vectors, then a 3-element scalar tail
    print(f"tree reduce R=2 n={n}", flush=True)
    reps = [_randn(n, 11 + r, 1e-3) for r in range(2)]
    out = torch.empty(n, device="cuda")
    br.repro_tree_reduce(reps, out=out)
    torch.cuda.synchronize()
    for lo in (0, (1 << 31) - 2048, n - 4099, n - 3):
        hi = min(n, lo + 4099)
        ref = oracle.tree_reduce([to_host(r[lo:hi]) for r in reps])
        assert_bitwise(to_host(out[lo:hi]), ref, f"window [{lo}, {hi})")


def test_gemm_output_past_two_to_the_31():
    M = N = 46341  # M * N = 2,147,488,281 > 2^31 - 1; 46341 = 362 * 128 + 5
    K = 3
    print(f"gemm {M}x{N}x{K}", flush=True)
    A = _randn(M * K, 21, 1.0).view(M, K)
    B = _randn(K * N, 22, 1.0).view(K, N)
    C = br.repro_gemm(A, B)
    torch.cuda.synchronize()
    Ah, Bh = to_host(A), to_host(B)
    for r in (0, 1, 40000, M - 5, M - 1):
        assert_bitwise(to_host(C[r]), oracle.gemm(Ah[r:r + 1], Bh)[0], f"row {r}")
    for c in (0, N - 6, N - 1):
        assert_bitwise(to_host(C[:, c]), oracle.gemm(Ah, np.ascontiguousarray(Bh[:, c:c + 1]))[:, 0], f"column {c}")


def test_gemm_slab_offsets_past_two_to_the_32_bytes():
    # A is a 512 x 48 view with a leading dimension of 2^22 + 4 floats (8.6 GB
    # spanned), so a lane's byte offset inside one 256-row slab of A passes
    # 2^32: the interior tiles cannot use 32-bit slab offsets and take the
    # bounds-checked loads.  The result must equal the same product from a
    # compact copy of A (interior loads) word for word, and the oracle's rows.
    M, K, N = 512, 48, 32768  # 2 x 256 tiles of 256 x 128: the large-output kernel
    lda = (1 << 22) + 4
    print(f"gemm {M}x{N}x{K} lda={lda}", flush=True)
    compact = _randn(M * K, 41, 1.0).view(M, K)
    big = torch.empty((M - 1) * lda + K, device="cuda")
    A = big.as_strided((M, K), (lda, 1))
    A.copy_(compact)
    B = _randn(K * N, 42, 1.0).view(K, N)
    C_view = br.repro_gemm(A, B)
    C_compact = br.repro_gemm(compact, B)
    torch.cuda.synchronize()
    assert torch.equal(C_view.view(torch.int32), C_compact.view(torch.int32))
    Ah, Bh = to_host(compact), to_host(B)
    for r in (0, 255, 256, M - 1):
        assert_bitwise(to_host(C_view[r]), oracle.gemm(Ah[r:r + 1], Bh)[0], f"row {r}")
    del big


def test_state_hash_past_two_to_the_32_words():
    n = (1 << 32) + 1000  # 17.2 GB; the last leaf holds 4,000 bytes
    print(f"state hash n_words={n}", flush=True)
    words = _randn(n, 31, 0.02)
    ws = br.hash_workspace(n)
    digest = torch.empty(32, dtype=torch.uint8, device="cuda")
    br.repro_state_hash_async(words, digest, ws)
    again = torch.empty(32, dtype=torch.uint8, device="cuda")
    br.repro_state_hash_async(words, again, ws)
    torch.cuda.synchronize()
    assert torch.equal(digest, again)
    leaves = (4 * n + 4095) // 4096
    level0 = ws[:32 * leaves].view(leaves, 32)
    for leaf in (0, 1, (1 << 22) - 1, 1 << 22, leaves - 2, leaves - 1):
        w = to_host(words[leaf * 1024:min(n, (leaf + 1) * 1024)])
        ref = oracle.state_hash_one_leaf(w, leaf, leaf == leaves - 1)
        assert to_host(level0[leaf]).tobytes() == ref, f"leaf {leaf}"
