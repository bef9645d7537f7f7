"""Pins for the oracle TreeFold reduction (CPU only).

OPEN-1B paper, Appendix A.1 with Algorithm 2 (TreeFold Push/Result), section 5
("The deterministic all-reduce": recursive-doubling butterfly; non-power-of-two
counts fold into the largest power-of-two block plus a remainder), section 6
with Algorithm 1, and Appendix A.3 (averages as a multiply by a host-computed
reciprocal).
"""
import itertools

import numpy as np
import pytest

import oracle


def test_integer_sums_exact_power_of_two_average():
    # Small integers: every partial sum is exact, and x * fl(1/R) is exact for
    # R a power of two, so the result is the exact mean.
    rng = np.random.default_rng(1)
    for R in (1, 2, 4, 8, 16, 32):
        reps = [rng.integers(-1000, 1001, size=513).astype(np.float32) for _ in range(R)]
        exact = np.sum(np.stack(reps).astype(np.int64), axis=0)
        out = oracle.tree_reduce(reps, average=True)
        np.testing.assert_array_equal(out.astype(np.float64), exact / R)


def test_integer_sums_exact_any_count():
    rng = np.random.default_rng(2)
    for R in (3, 5, 6, 7, 9, 13, 31, 64):
        reps = [rng.integers(-1000, 1001, size=257).astype(np.float32) for _ in range(R)]
        exact = np.sum(np.stack(reps).astype(np.int64), axis=0)
        out = oracle.tree_reduce(reps, average=False)
        np.testing.assert_array_equal(out.astype(np.int64), exact)


def _butterfly(reps):
    """Recursive-doubling all-reduce over R = 2^k ranks, emulated in binary32.

    At hop h every rank r exchanges its whole buffer with rank r ^ 2^h and both
    compute (lower rank's buffer) + (higher rank's buffer)."""
    R = len(reps)
    bufs = [np.asarray(r, np.float32).copy() for r in reps]
    h = 1
    while h < R:
        new = []
        for r in range(R):
            p = r ^ h
            lo, hi = (bufs[r], bufs[p]) if r < p else (bufs[p], bufs[r])
            new.append((lo + hi).astype(np.float32))
        bufs = new
        h <<= 1
    for r in range(1, R):
        assert bufs[r].tobytes() == bufs[0].tobytes()
    return bufs[0]


@pytest.mark.parametrize("R", [2, 4, 8, 16])
def test_treefold_equals_recursive_doubling(R):
    # Appendix A.1: TreeFold reproduces the cluster's recursive-doubling
    # pairing (lower replica on the left) bit for bit.
    rng = np.random.default_rng(R)
    n = 20_000
    reps = []
    for _ in range(R):
        x = rng.standard_normal(n) * 1e-3
        mask = rng.random(n) < 0.01
        x[mask] = rng.standard_normal(mask.sum()) * 10
        reps.append(x.astype(np.float32))
    out = oracle.tree_reduce(reps, average=False)
    assert out.tobytes() == _butterfly(reps).tobytes()


def test_non_power_of_two_remainder_folded_first():
    # R = 7 = 4 + 2 + 1.  Algorithm 2's Result starts from the lowest-level
    # entry (x6) and adds the rest in ascending level: (x6 + (x4+x5)) +
    # ((x0+x1)+(x2+x3)), i.e. the remainder block is folded before it meets
    # the largest power-of-two block (section 5).  With
    # x = [2^24, 0, 0, 0, 1, 0, 1] that is 2 + 2^24 = 2^24 + 2 exactly, while
    # folding the largest block first, (2^24 + 1) + 1, gives 2^24 (two ties
    # to even).
    x = np.array([2.0 ** 24, 0, 0, 0, 1, 0, 1], np.float32)
    reps = [np.array([v], np.float32) for v in x]
    assert oracle.tree_reduce(reps, average=False)[0] == np.float32(2.0 ** 24 + 2)
    # With the average: fl((2^24 + 2) * fl(1/7)).
    r7 = np.float32(1.0) / np.float32(7.0)
    assert oracle.tree_reduce(reps, average=True)[0] == np.float32(np.float32(2.0 ** 24 + 2) * r7)


def test_three_and_five_and_six_groupings():
    # R = 3: x2 + (x0 + x1).  With [2^24, 1, 1]: (2^24+1) -> 2^24, + 1 -> 2^24.
    # A flat left-to-right loop gives the same here, so also check [1, 1, 2^24]:
    # tree: (1+1) + 2^24 = 2^24 + 2.
    reps = [np.array([v], np.float32) for v in (1.0, 1.0, 2.0 ** 24)]
    assert oracle.tree_reduce(reps, average=False)[0] == np.float32(2.0 ** 24 + 2)
    # R = 6 = 4 + 2: (x4 + x5) + ((x0+x1)+(x2+x3)).  With x = [2^24,1,0,0,1,0]:
    # x0+x1 -> 2^24, S0123 = 2^24; S45 = 1; 1 + 2^24 -> 2^24.
    reps = [np.array([v], np.float32) for v in (2.0 ** 24, 1, 0, 0, 1, 0)]
    assert oracle.tree_reduce(reps, average=False)[0] == np.float32(2.0 ** 24)
    # ...and [1, 0, 0, 1, 2^24, 2]: S0123 = 2, S45 = 2^24 + 2; sum 2^24 + 4.
    reps = [np.array([v], np.float32) for v in (1, 0, 0, 1, 2.0 ** 24, 2)]
    assert oracle.tree_reduce(reps, average=False)[0] == np.float32(2.0 ** 24 + 4)


@pytest.mark.parametrize("R", [3, 5, 6, 7])
def test_average_is_reciprocal_multiply_not_division(R):
    # Appendix A.3: for a divisor that is not a power of two, fl(x * fl(1/R))
    # and fl(x / R) differ by up to one ulp for some x.  Find such an x; the
    # oracle must give the reciprocal-multiply value.
    rR = np.float32(1.0) / np.float32(R)
    rng = np.random.default_rng(R)
    x = (rng.standard_normal(200_000)).astype(np.float32)
    mul = (x * rR).astype(np.float32)
    div = (x / np.float32(R)).astype(np.float32)
    differ = np.nonzero(mul != div)[0]
    assert differ.size > 0
    xs = x[differ[:64]]
    reps = [xs] + [np.zeros_like(xs) for _ in range(R - 1)]  # exact sum = xs
    out = oracle.tree_reduce(reps, average=True)
    np.testing.assert_array_equal(out, mul[differ[:64]])
    assert (out != div[differ[:64]]).all()
    # The differences are at most one ulp.
    assert (np.abs(out.view(np.int32).astype(np.int64) - div[differ[:64]].view(np.int32)) <= 1).all()


def test_resident_partials_bound():
    # Appendix A.1: at most floor(log2 R) + 1 partials resident, "at most 4"
    # at R = 8.
    for R in range(1, 40):
        reps = [np.full(3, float(r), np.float32) for r in range(R)]
        _, resident = oracle.tree_reduce(reps, average=False, return_resident=True)
        assert resident == int(np.floor(np.log2(R))) + 1
    _, resident = oracle.tree_reduce([np.zeros(2, np.float32)] * 8, return_resident=True)
    assert resident == 4


def _all_trees(leaves):
    """Every full binary tree over an ordered list of leaf indices."""
    if len(leaves) == 1:
        yield leaves[0]
        return
    for split in range(1, len(leaves)):
        for lt in _all_trees(leaves[:split]):
            for rt in _all_trees(leaves[split:]):
                yield (lt, rt)


def _eval(tree, vals):
    if isinstance(tree, tuple):
        return np.float32(_eval(tree[0], vals) + _eval(tree[1], vals))
    return vals[tree]


@pytest.mark.parametrize("R", [3, 4, 5, 6])
def test_tree_shape_changes_bits(R):
    # Non-vacuity: on data shaped like the workloads (N(0,1e-3) with a few
    # large outliers) different groupings and orders of the same addends give
    # different binary32 sums, so parity on such data can tell TreeFold from
    # other orders.
    rng = np.random.default_rng(100 + R)
    trees = [t for perm in itertools.permutations(range(R)) for t in _all_trees(list(perm))]
    discriminating = 0
    for _ in range(50):
        vals = rng.standard_normal(R) * 1e-3
        vals[rng.integers(0, R)] *= 1e4
        vals = vals.astype(np.float32)
        if len({_eval(t, vals).tobytes() for t in trees}) > 1:
            discriminating += 1
    assert discriminating > 10


def test_r1_and_empty():
    x = np.array([1.5, -2.0, 2.0 ** -130], np.float32)  # last one subnormal: reads as +0
    out = oracle.tree_reduce([x], average=True)
    np.testing.assert_array_equal(out, np.array([1.5, -2.0, 0.0], np.float32))
    # One replica without the average is no operation at all: the words copy.
    out = oracle.tree_reduce([x], average=False)
    assert out.tobytes() == x.tobytes()
    assert oracle.tree_reduce([np.zeros(0, np.float32)] * 3).size == 0
