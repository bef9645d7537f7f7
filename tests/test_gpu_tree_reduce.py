"""GPU parity: repro_tree_reduce against the oracle TreeFold, word for word.

OPEN-1B paper, Appendix A.1 (Algorithm 2) and Appendix A.3.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu


def _replicas(R, n, seed=0, offset_tid=0x7000):
    return [synth.generate(n, synth.OUTLIER_SCALED, offset_tid + 64 * seed + r, 1e-3, 0.01, 1e4) for r in range(R)]


@pytest.mark.parametrize("R", list(range(1, 17)) + [31, 33, 63, 64])
def test_every_replica_count(R):
    n = 4099  # ragged: not a multiple of 4 or of the block size
    reps = _replicas(R, n, seed=R)
    dreps = [to_dev(x) for x in reps]
    for average in (True, False):
        ref = oracle.tree_reduce(reps, average=average)
        for variant in (0, 1, 2):
            out = br.repro_tree_reduce(dreps, average=average, variant=variant)
            assert_bitwise(to_host(out), ref, f"R={R} average={average} variant={variant}")


def test_tiny_workload():
    cfg = synth.TINY
    reps = [synth.tiny_replica(r) for r in range(cfg["R"])]
    ref = oracle.tree_reduce(reps)
    out = br.repro_tree_reduce([to_dev(x) for x in reps])
    assert_bitwise(to_host(out), ref, "tiny reduce")


def test_gradient_reduction_workload_full_size():
    # R = 8 replicas of 16,777,216 floats, 0.1% outliers ~N(0,10); every word
    # of the output is compared, and ten repeats give the same bytes.
    cfg = synth.REDUCE
    print(f"reduce workload R={cfg['R']} n={cfg['n']}", flush=True)
    reps = [synth.reduce_replica(r) for r in range(cfg["R"])]
    ref = oracle.tree_reduce(reps)
    dreps = [to_dev(x) for x in reps]
    out = br.repro_tree_reduce(dreps)
    assert_bitwise(to_host(out), ref, "reduce workload")
    first = out.clone()
    for _ in range(10):
        again = br.repro_tree_reduce(dreps)
        assert torch.equal(again.view(torch.int32), first.view(torch.int32))


def test_non_power_of_two_grouping_witness():
    # R = 7: the remainder (x6 + (x4 + x5)) is folded before the largest
    # block, so [2^24, 0, 0, 0, 1, 0, 1] sums to 2^24 + 2.
    x = [np.full(8, v, np.float32) for v in (2.0 ** 24, 0, 0, 0, 1, 0, 1)]
    out = br.repro_tree_reduce([to_dev(v) for v in x], average=False)
    assert (to_host(out) == np.float32(2.0 ** 24 + 2)).all()


def test_in_place_output_and_unaligned_views():
    R, n = 5, 10_001
    reps = _replicas(R, n + 1, seed=99)
    ref = oracle.tree_reduce([r[1:] for r in reps])
    # Views that start one float into their allocation: 4-byte, not 16-byte
    # aligned, so the scalar kernel runs.
    dbase = [to_dev(x) for x in reps]
    views = [d[1:] for d in dbase]
    out = br.repro_tree_reduce(views)
    assert_bitwise(to_host(out), ref, "unaligned")
    # Output aliasing replica 0.
    dreps = [to_dev(x[1:].copy()) for x in reps]
    br.repro_tree_reduce(dreps, out=dreps[0])
    assert_bitwise(to_host(dreps[0]), ref, "in place")


def test_flush_of_subnormal_inputs_and_results():
    # Subnormal inputs read as zero; sums that are exactly subnormal flush.
    tiny = np.float32(2.0 ** -127)  # subnormal
    a = np.array([tiny, 1.5 * 2.0 ** -126, 2.0 ** -126, -tiny, 1.0], np.float32)
    b = np.array([tiny, -(2.0 ** -126), -1.5 * 2.0 ** -126, -0.0, tiny], np.float32)
    ref = oracle.tree_reduce([a, b], average=False)
    out = br.repro_tree_reduce([to_dev(a), to_dev(b)], average=False)
    assert_bitwise(to_host(out), ref, "flush")
    assert to_host(out).view(np.uint32).tolist() == [0, 0, 0x80000000, 0x80000000, 0x3F800000]


def test_empty_and_errors():
    d = torch.zeros(4, device="cuda")
    out = torch.zeros(0, device="cuda")
    br.repro_tree_reduce([torch.zeros(0, device="cuda")] * 3, out=out)
    with pytest.raises(ValueError):
        br.repro_tree_reduce([d] * 65)
    lib = br.library()
    import ctypes
    ptrs = (ctypes.c_void_p * 2)(d.data_ptr(), d.data_ptr() + 2)  # second pointer misaligned
    assert lib.repro_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 2, 1, d.data_ptr(), 1, None) == -2
    assert lib.repro_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 0, 4, d.data_ptr(), 1, None) == -1
