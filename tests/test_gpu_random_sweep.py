"""GPU parity on a seeded sweep of random shapes, layouts and offsets.

Each case draws its sizes, transposes, leading-dimension padding and base
offsets (so 16-byte and 4-byte aligned views both occur) from a fixed seed,
runs every kernel variant of the operation and compares every output word
with the oracle.  Covers the unfused GEMM (all four variants), the fused
convention (both units), TreeFold, AdamW and the state hash.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = 24


def _view(host, rows, cols, ld, off):
    """A rows x cols device view with leading dimension ld at element offset off."""
    buf = np.zeros(off + max(rows - 1, 0) * ld + cols + 4, np.float32)
    for r in range(rows):
        buf[off + r * ld: off + r * ld + cols] = host[r]
    d = to_dev(buf)
    return torch.as_strided(d, (rows, cols), (ld, 1), off)


@pytest.mark.parametrize("case", range(CASES))
def test_gemm_random_layouts(case):
    rng = np.random.default_rng(1000 + case)
    M, N, K = (int(x) for x in rng.integers(1, 300, 3))
    if case % 6 == 0:
        K = int(rng.integers(0, 3))
    ta, tb = (bool(x) for x in rng.integers(0, 2, 2))
    A = synth.generate(M * K, synth.NORMAL, synth.tid(0x0D, case), 1.0).reshape(M, K)
    B = synth.generate(K * N, synth.STUDENT_T3, synth.tid(0x0E, case), 1.0).reshape(K, N)
    As = np.ascontiguousarray(A.T) if ta else A
    Bs = np.ascontiguousarray(B.T) if tb else B
    pad = [int(x) for x in rng.integers(0, 9, 3)]
    off = [int(x) for x in rng.integers(0, 4, 3)]
    dA = _view(As, As.shape[0], As.shape[1], As.shape[1] + pad[0], off[0])
    dB = _view(Bs, Bs.shape[0], Bs.shape[1], Bs.shape[1] + pad[1], off[1])
    ref = oracle.gemm(As, Bs, ta, tb)
    ref_f = oracle.gemm(As, Bs, ta, tb, fused=True)
    what = f"M={M} N={N} K={K} ta={ta} tb={tb} pad={pad} off={off}"
    for variant in (0, 1, 2, 3, 4):
        out = _view(np.full((M, N), 7.0, np.float32), M, N, N + pad[2], off[2])
        br.repro_gemm(dA, dB, ta, tb, out=out, variant=variant)
        assert_bitwise(to_host(out), ref, f"{what} variant={variant}")
    for variant in (0, 1):
        out = _view(np.full((M, N), 7.0, np.float32), M, N, N + pad[2], off[2])
        br.repro_gemm_fma(dA, dB, ta, tb, out=out, variant=variant)
        assert_bitwise(to_host(out), ref_f, f"{what} fused variant={variant}")


@pytest.mark.parametrize("case", range(CASES))
def test_reduce_adamw_hash_random_sizes(case):
    rng = np.random.default_rng(2000 + case)
    R = int(rng.integers(1, 65))
    n = int(rng.integers(0, 20000))
    off = int(rng.integers(0, 4))
    reps = [synth.generate(n, synth.OUTLIER_REPLACE, synth.tid(0x0F, r), 1e-3, 0.01, 10.0) for r in range(R)]
    dreps = [to_dev(np.concatenate([np.zeros(off, np.float32), x]))[off:] for x in reps]
    ref = oracle.tree_reduce(reps)
    for variant in (0, 1, 2):
        out = br.repro_tree_reduce(dreps, variant=variant)
        assert_bitwise(to_host(out), ref, f"R={R} n={n} off={off} variant={variant}")
    step = int(rng.integers(1, 2000))
    w = synth.generate(n, synth.NORMAL, synth.tid(0x10, case), 0.02)
    m = synth.generate(n, synth.NORMAL, synth.tid(0x11, case), 1e-4)
    v = synth.generate(n, synth.HALF_NORMAL, synth.tid(0x12, case), 1e-6)
    st = np.concatenate([w, m, v])
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=step)
    want = oracle.adamw(st, ref, **hp)
    for variant in (0, 1):
        d = to_dev(np.concatenate([np.zeros(off, np.float32), st]))[off:]
        br.repro_adamw(d, to_dev(ref), variant=variant, **hp)
        assert_bitwise(to_host(d), want, f"adamw n={n} off={off} step={step} variant={variant}")
    d = to_dev(np.concatenate([np.zeros(off, np.float32), want]))[off:]
    assert br.repro_state_hash(d) == oracle.state_hash(want), f"hash n={n} off={off}"
