"""Calls from several host threads at once, each on its own stream.

The library keeps no per-call host state except the side streams and
events of the pipelined AdamW + hash form, whose enqueue sequence runs
under a lock; ctypes releases the interpreter lock during each call, so the
calls below really overlap.  Every thread must reproduce the result of the
same calls made from one thread, bit for bit.
"""
import threading

import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import synth
from parity_util import to_dev, to_host

pytestmark = pytest.mark.gpu

N = 1 << 20  # 1024 leaves per region; chunk 2^18 gives four pipelined chunks
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _inputs(k):
    reps = [synth.generate(N, synth.NORMAL, synth.tid(9, 0x40 + 8 * k + r), 1e-3) for r in range(4)]
    state = np.concatenate([synth.generate(N, synth.NORMAL, synth.tid(9, 0x60 + k), 0.02),
                            np.zeros(2 * N, np.float32)])
    return reps, state


def _run(reps_d, state0, chunk, rounds, out):
    """reduce -> AdamW + hash (fused or pipelined), `rounds` times, on the current stream."""
    g = torch.empty(N, device="cuda")
    st = to_dev(state0)
    ws = br.hash_workspace(3 * N)
    digest = torch.empty(32, dtype=torch.uint8, device="cuda")
    digests = []
    for step in range(1, rounds + 1):
        br.repro_tree_reduce(reps_d, out=g)
        br.repro_adamw_hash(st, g, digest, ws, step=step, chunk=chunk, **HP)
        digests.append(digest.clone())
    torch.cuda.current_stream().synchronize()
    out["state"] = to_host(st)
    out["digests"] = [bytes(to_host(d).tobytes()) for d in digests]


@pytest.mark.parametrize("chunk", [0, 1 << 18])
def test_threads_on_separate_streams_match_one_thread(chunk):
    rounds = 6
    work = [_inputs(k) for k in range(2)]
    reps_d = [[to_dev(x) for x in reps] for reps, _ in work]
    refs = []
    for k in range(2):
        ref = {}
        _run(reps_d[k], work[k][1], chunk, rounds, ref)
        refs.append(ref)
    results = [dict() for _ in range(4)]
    errors = []

    def worker(t):
        try:
            k = t % 2
            with torch.cuda.stream(torch.cuda.Stream()):
                _run(reps_d[k], work[k][1], chunk, rounds, results[t])
        except Exception as e:  # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for t in range(4):
        k = t % 2
        assert np.array_equal(results[t]["state"].view(np.uint32), refs[k]["state"].view(np.uint32)), f"thread {t}"
        assert results[t]["digests"] == refs[k]["digests"], f"thread {t} digests"
