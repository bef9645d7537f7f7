"""Pins for the oracle's Algorithm 1 replay reduction and the streaming TreeFold (CPU only).

OPEN-1B paper, section 6 (Algorithm 1: microbatch accumulation, the
ascending-shard running sum, the TreeFold push per replica, averages) and
Appendix A.1-A.3 (TreeFold; every average is a multiply by a host-computed
reciprocal).
"""
import numpy as np
import pytest

import oracle


def _grads(N, accum, n, seed, integer=False):
    rng = np.random.default_rng(seed)
    if integer:
        return [rng.integers(-64, 65, n).astype(np.float32) for _ in range(N * accum)]
    out = []
    for _ in range(N * accum):
        x = rng.standard_normal(n) * 1e-3
        m = rng.random(n) < 0.01
        x[m] *= 1e4
        out.append(x.astype(np.float32))
    return out


@pytest.mark.parametrize("rep,shard,accum", [(1, 1, 1), (2, 4, 2), (8, 4, 4), (4, 8, 1), (1, 2, 8)])
def test_integer_gradients_give_the_exact_mean(rep, shard, accum):
    # Small integers and power-of-two counts: every product by a reciprocal
    # and every partial sum is exact, so the result is the exact mean of all
    # rep * shard * accum microbatch gradients.
    n = 300
    grads = _grads(rep * shard, accum, n, 1, integer=True)
    exact = np.sum(np.stack(grads).astype(np.float64), axis=0) / (rep * shard * accum)
    out = oracle.replay_reduce(grads, rep, shard, accum)
    np.testing.assert_array_equal(out.astype(np.float64), exact)


def test_shards_are_summed_in_ascending_order():
    # One replica, three shards, one microbatch: inner = (g0 + g1) + g2.
    # With [2^24, 1, 1]: 2^24 + 1 -> 2^24 (tie to even), + 1 -> 2^24; any
    # order that adds the two 1s first gives 2^24 + 2.
    grads = [np.array([v], np.float32) for v in (2.0 ** 24, 1.0, 1.0)]
    r3 = np.float32(1) / np.float32(3)
    out = oracle.replay_reduce(grads, 1, 3, 1)
    assert out[0] == np.float32(np.float32(2.0 ** 24) * r3)


def test_microbatches_accumulate_left_to_right_after_scaling():
    # accum = 4: g = (((0 + x0/4) + x1/4) + x2/4) + x3/4 with each /4 exact.
    # x = [2^26, 4, 4, -2^26] -> terms [2^24, 1, 1, -2^24]: 2^24 + 1 -> 2^24,
    # + 1 -> 2^24, - 2^24 -> 0.  Summing first and scaling after, or any
    # other order, gives 2.
    grads = [np.array([v], np.float32) for v in (2.0 ** 26, 4.0, 4.0, -(2.0 ** 26))]
    assert oracle.replay_reduce(grads, 1, 1, 4)[0] == 0.0


def test_buffers_are_rank_major_then_microbatch():
    # dp_shard = 2 ranks, accum = 2: buffers [r0k0, r0k1, r1k0, r1k1].  With
    # [2^25, 2, -2^25, 2] the halves are [2^24, 1, -2^24, 1]:
    # g0 = 2^24 + 1 -> 2^24, g1 = -2^24 + 1 (exact), inner = 1, result 0.5.
    # Pairing microbatch-major ([r0k0, r1k0], [r0k1, r1k1]) gives
    # (2^24 - 2^24) + (1 + 1) = 2 and a result of 1.
    grads = [np.array([v], np.float32) for v in (2.0 ** 25, 2.0, -(2.0 ** 25), 2.0)]
    assert oracle.replay_reduce(grads, 1, 2, 2)[0] == np.float32(0.5)


def test_every_average_is_a_reciprocal_multiply():
    # accum = 3 with a single microbatch term per rank would not exercise the
    # sum; use accum = 3 with two zero microbatches: g = fl(x * fl(1/3)),
    # which differs from fl(x / 3) for some x (Appendix A.3).
    rng = np.random.default_rng(7)
    x = rng.standard_normal(100_000).astype(np.float32)
    r3 = np.float32(1) / np.float32(3)
    want = (x * r3).astype(np.float32)
    differ = want != (x / np.float32(3)).astype(np.float32)
    assert differ.any()
    grads = [x, np.zeros_like(x), np.zeros_like(x)]
    out = oracle.replay_reduce(grads, 1, 1, 3)
    np.testing.assert_array_equal(out, want)
    # dp_shard = 3: inner * fl(1/3); dp_replicate = 3: Result * fl(1/3).
    z = np.zeros_like(x)
    np.testing.assert_array_equal(oracle.replay_reduce([x, z, z], 1, 3, 1), want)
    np.testing.assert_array_equal(oracle.replay_reduce([x, z, z], 3, 1, 1), want)


@pytest.mark.parametrize("rep", [1, 2, 3, 5, 7, 8, 13])
def test_one_shard_one_microbatch_is_the_replica_treefold(rep):
    # Algorithm 1 reduces to the inter-node TreeFold when each replica is a
    # single rank with a single microbatch.
    grads = _grads(rep, 1, 4099, 100 + rep)
    np.testing.assert_array_equal(oracle.replay_reduce(grads, rep, 1, 1), oracle.tree_reduce(grads, average=True))


@pytest.mark.parametrize("R", list(range(1, 21)))
def test_streaming_push_result_equals_treefold(R):
    n = 777
    parts = _grads(R, 1, n, 300 + R)
    depth = int(np.floor(np.log2(R))) + 1
    slots = [np.full(n, np.nan, np.float32) for _ in range(depth)]
    for i, p in enumerate(parts):
        oracle.fold_push(slots, i, p)
    # Only floor(log2 R) + 1 slots are ever written (the list has no more),
    # and every level whose bit is set in R holds a partial.  A consumed slot
    # keeps stale data, which Result never reads.
    for L in range(depth):
        if (R >> L) & 1:
            assert not np.isnan(slots[L]).any()
    np.testing.assert_array_equal(oracle.fold_result(slots, R, 0), oracle.tree_reduce(parts, average=False))
    np.testing.assert_array_equal(oracle.fold_result(slots, R, R), oracle.tree_reduce(parts, average=True))
