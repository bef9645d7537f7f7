"""GPU parity: repro_state_hash against the oracle BLAKE2b tree hash.

OPEN-1B paper, Appendix B and Figure 11 (BLAKE2b state hash); section 3.2
(state hashed in FP32).
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [0, 1, 2, 3, 31, 32, 33, 1023, 1024, 1025, 16 * 1024, 16 * 1024 + 1, 33 * 1024 + 7,
                               16 * 16 * 1024 + 5, 5000 * 1024, 300 * 16 * 1024 + 3])
def test_sizes(n):
    w = synth.generate(n, synth.NORMAL, 0xA000 + n % 251, 1.0) if n else np.zeros(0, np.float32)
    ref = oracle.state_hash(w)
    d = to_dev(w) if n else torch.zeros(0, device="cuda")
    assert br.repro_state_hash(d) == ref, f"n={n}"


def test_unaligned_input():
    n = 16 * 1024 + 9
    w = synth.generate(n + 1, synth.NORMAL, 0xA100, 1.0)
    d = to_dev(w)[1:]  # 4-byte aligned only
    assert br.repro_state_hash(d) == oracle.state_hash(w[1:])


def test_workspace_size_and_errors():
    lib = br.library()
    for n in (0, 1, 1024, 10 ** 6):
        assert br.repro_state_hash_workspace_bytes(n) > 0
    d = torch.zeros(1024, device="cuda")
    ws = torch.zeros(br.repro_state_hash_workspace_bytes(1024), dtype=torch.uint8, device="cuda")
    dig = torch.zeros(32, dtype=torch.uint8, device="cuda")
    assert lib.repro_state_hash(d.data_ptr(), 1024, ws.data_ptr(), ws.numel() - 1, dig.data_ptr(), None) == -4
    assert lib.repro_state_hash(d.data_ptr(), -1, ws.data_ptr(), ws.numel(), dig.data_ptr(), None) == -1


def test_single_bit_flip_changes_the_digest():
    w = synth.generate(65536 * 3, synth.NORMAL, 0xA200, 1.0)
    d = to_dev(w)
    h0 = br.repro_state_hash(d)
    d.view(torch.int32)[77_777] ^= 1
    h1 = br.repro_state_hash(d)
    assert h0 != h1
    w2 = w.copy()
    w2.view(np.uint32)[77_777] ^= 1
    assert h1 == oracle.state_hash(w2)


def test_tiny_workload_state():
    # The [w | m | v] of the tiny chained step (reduce, then AdamW at step 1).
    cfg = synth.TINY
    reps = [synth.tiny_replica(r) for r in range(cfg["R"])]
    g = br.repro_tree_reduce([to_dev(x) for x in reps])
    n = cfg["n"]
    state = np.concatenate([synth.tiny_adamw_weights(n), np.zeros(2 * n, np.float32)])
    hp = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"], weight_decay=cfg["wd"])
    st = to_dev(state)
    br.repro_adamw(st, g, step=cfg["step"], **hp)
    ref_state = oracle.adamw(state, oracle.tree_reduce(reps), step=cfg["step"], **hp)
    assert br.repro_state_hash(st) == oracle.state_hash(ref_state)


def test_optimizer_workload_state_full_size():
    # 14.4 GB: [w | m | v] of n = 1.2e9, hashed on the GPU ten times and once
    # by the oracle (single-threaded BLAKE2b over every byte).
    cfg = synth.ADAMW
    n = cfg["n"]
    print(f"hash workload n_words={3 * n}", flush=True)
    host = np.empty(3 * n, np.float32)
    synth.adamw_w(n, out=host[:n])
    synth.adamw_m(n, out=host[n:2 * n])
    synth.adamw_v(n, out=host[2 * n:])
    d = torch.from_numpy(host).cuda()
    ws = br.hash_workspace(3 * n)
    first = br.repro_state_hash(d, ws)
    for _ in range(9):
        assert br.repro_state_hash(d, ws) == first
    print("gpu digest", first.hex(), flush=True)
    assert first == oracle.state_hash(host)
