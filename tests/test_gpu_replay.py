"""GPU parity: repro_replay_reduce and the streaming TreeFold against the oracle.

OPEN-1B paper, section 6 (Algorithm 1) and Appendix A.1-A.3.
"""
import ctypes

import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu


def _grads(nbuf, n, tid0):
    return [synth.generate(n, synth.OUTLIER_SCALED, tid0 + b, 1e-3, 0.01, 1e4) for b in range(nbuf)]


@pytest.mark.parametrize("rep,shard,accum", [(1, 1, 1), (1, 3, 1), (2, 2, 2), (3, 5, 3), (8, 4, 2), (7, 1, 4),
                                             (5, 8, 1), (64, 1, 1), (13, 2, 3),
                                             (64, 6, 1), (8, 8, 6)])  # the last two: REPRO_MAX_REPLAY_BUFFERS = 384
def test_layouts(rep, shard, accum):
    n = 4099  # ragged tail after the 16-byte vectors
    grads = _grads(rep * shard * accum, n, 0xB000 + 97 * rep + 13 * shard + accum)
    ref = oracle.replay_reduce(grads, rep, shard, accum)
    out = br.repro_replay_reduce([to_dev(g) for g in grads], rep, shard, accum)
    assert_bitwise(to_host(out), ref, f"replay {rep}x{shard}x{accum}")


def test_open1b_main_phase_layout():
    # 6 nodes x 8 shards per node x 6 microbatches per rank = 288 gradient
    # buffers (the main-phase layout: 288 microbatches per step on 48 GPUs).
    rep, shard, accum, n = 6, 8, 6, 1 << 18
    print(f"replay {rep}x{shard}x{accum} n={n}", flush=True)
    grads = _grads(rep * shard * accum, n, 0xB800)
    ref = oracle.replay_reduce(grads, rep, shard, accum)
    dg = [to_dev(g) for g in grads]
    out = br.repro_replay_reduce(dg, rep, shard, accum)
    assert_bitwise(to_host(out), ref, "main-phase layout")
    again = br.repro_replay_reduce(dg, rep, shard, accum)
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))


def test_witnesses_and_unaligned():
    # Ascending shards: (2^24 + 1) + 1 -> 2^24, then x fl(1/3).
    g = [to_dev(np.full(9, v, np.float32)) for v in (2.0 ** 24, 1.0, 1.0)]
    r3 = np.float32(1) / np.float32(3)
    assert (to_host(br.repro_replay_reduce(g, 1, 3, 1)) == np.float32(np.float32(2.0 ** 24) * r3)).all()
    # Rank-major buffers: [2^25, 2, -2^25, 2] with shard 2, accum 2 -> 0.5.
    g = [to_dev(np.full(5, v, np.float32)) for v in (2.0 ** 25, 2.0, -(2.0 ** 25), 2.0)]
    assert (to_host(br.repro_replay_reduce(g, 1, 2, 2)) == np.float32(0.5)).all()
    # 4-byte aligned views take the scalar kernel.
    grads = _grads(6, 1001, 0xB900)
    ref = oracle.replay_reduce([x[1:] for x in grads], 3, 2, 1)
    views = [to_dev(x)[1:] for x in grads]
    assert_bitwise(to_host(br.repro_replay_reduce(views, 3, 2, 1)), ref, "unaligned")


def test_out_may_be_one_of_the_buffers():
    grads = _grads(12, 2051, 0xB950)
    ref = oracle.replay_reduce(grads, 2, 3, 2)
    dg = [to_dev(g) for g in grads]
    for j in (0, 7, 11):
        dg[j] = to_dev(grads[j])
        out = br.repro_replay_reduce(dg, 2, 3, 2, out=dg[j])
        assert out.data_ptr() == dg[j].data_ptr()
        assert_bitwise(to_host(out), ref, f"out aliases buffer {j}")
        dg[j] = to_dev(grads[j])


def test_push_into_the_free_slot():
    # `part` may already sit in the slot it will be stored to.
    n, R = 3001, 11
    parts = _grads(R, n, 0xB970)
    slots = [torch.empty(n, device="cuda") for _ in range(4)]
    for i, p in enumerate(parts):
        t = (~i & (i + 1)).bit_length() - 1
        slots[t].copy_(to_dev(p))
        br.repro_fold_push(slots, i, slots[t])
    out = torch.empty(n, device="cuda")
    assert_bitwise(to_host(br.repro_fold_result(slots, R, out, divisor=R)), oracle.tree_reduce(parts), "in place")


@pytest.mark.parametrize("R", [1, 2, 3, 5, 7, 8, 13, 16, 31, 64, 127])  # 127: all seven slots in use
def test_streaming_fold(R):
    n = 10_001
    parts = _grads(R, n, 0xBA00 + R)
    depth = int(np.floor(np.log2(R))) + 1
    slots = [torch.empty(n, device="cuda") for _ in range(depth)]
    for i, p in enumerate(parts):
        br.repro_fold_push(slots, i, to_dev(p))
    out = torch.empty(n, device="cuda")
    assert_bitwise(to_host(br.repro_fold_result(slots, R, out)), oracle.tree_reduce(parts, average=False), "sum")
    assert_bitwise(to_host(br.repro_fold_result(slots, R, out, divisor=R)), oracle.tree_reduce(parts), "mean")


def test_errors():
    lib = br.library()
    d = torch.zeros(8, device="cuda")
    ptrs = (ctypes.c_void_p * 2)(d.data_ptr(), d.data_ptr())
    assert lib.repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 65, 1, 1, 8, d.data_ptr(), None) == -1
    assert lib.repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 1, 2, 0, 8, d.data_ptr(), None) == -1
    many = (ctypes.c_void_p * 385)(*([d.data_ptr()] * 385))
    assert lib.repro_replay_reduce(ctypes.cast(many, ctypes.c_void_p), 5, 7, 11, 8, d.data_ptr(), None) == -1  # 385
    assert lib.repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 1, 2, 1, 8, d.data_ptr() + 2, None) == -2
    slots = (ctypes.c_void_p * 7)(d.data_ptr(), None, None, None, None, None, None)
    assert lib.repro_fold_push(ctypes.cast(slots, ctypes.c_void_p), 1, d.data_ptr(), 8, None) == -1  # needs slot 1
    assert lib.repro_fold_result(ctypes.cast(slots, ctypes.c_void_p), 0, 8, d.data_ptr(), 0, None) == -1
