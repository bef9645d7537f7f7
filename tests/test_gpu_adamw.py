"""GPU parity: repro_adamw against the oracle AdamW step, word for word.

OPEN-1B paper, section 3.2 "Optimizer" and "Optimizer-state precision"; the
checkpoint page's flat [w | m | v] layout.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _state(n, tid):
    w = synth.generate(n, synth.NORMAL, tid, 0.02)
    m = synth.generate(n, synth.NORMAL, tid + 1, 1e-4)
    v = synth.generate(n, synth.HALF_NORMAL, tid + 2, 1e-6)
    g = synth.generate(n, synth.NORMAL, tid + 3, 1e-3)
    return np.concatenate([w, m, v]), g


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 65_536, 100_003])
@pytest.mark.parametrize("step", [1, 2, 7, 829, 830, 1000])
def test_sizes_steps_variants(n, step):
    state, g = _state(n, 0x9000 + n % 97)
    ref = oracle.adamw(state, g, step=step, **HP)
    for variant in (0, 1):
        st = to_dev(state)
        br.repro_adamw(st, to_dev(g), step=step, variant=variant, **HP)
        assert_bitwise(to_host(st), ref, f"n={n} step={step} variant={variant}")


def test_tiny_workload_chained_after_reduce():
    cfg = synth.TINY
    reps = [synth.tiny_replica(r) for r in range(cfg["R"])]
    g = br.repro_tree_reduce([to_dev(x) for x in reps])
    g_ref = oracle.tree_reduce(reps)
    n = cfg["n"]
    state = np.concatenate([synth.tiny_adamw_weights(n), np.zeros(2 * n, np.float32)])
    hp = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"], weight_decay=cfg["wd"])
    st = to_dev(state)
    br.repro_adamw(st, g, step=cfg["step"], **hp)
    assert_bitwise(to_host(st), oracle.adamw(state, g_ref, step=cfg["step"], **hp), "tiny adamw")


def test_directed_values():
    # Zero gradients and moments (u = 0/eps = 0), subnormal inputs (read as
    # zero), large and tiny magnitudes, sign changes.
    vals = np.array([0.0, -0.0, 2.0 ** -130, -(2.0 ** -130), 1e-30, -1e-30, 1e-3, -1e-3, 5.0, -5.0,
                     2.0 ** -126, 3e38, 1e-20], np.float32)
    n = vals.size ** 2
    w = np.repeat(vals, vals.size)
    g = np.tile(vals, vals.size)
    m = np.roll(w, 3)
    v = np.abs(np.roll(g, 5))
    state = np.concatenate([w, m, v]).astype(np.float32)
    for step in (1, 3):
        ref = oracle.adamw(state, g, step=step, **HP)
        st = to_dev(state)
        br.repro_adamw(st, to_dev(g), step=step, **HP)
        got = to_host(st)
        # g = 3e38 overflows g*g; every non-NaN word (infinities included)
        # must match, and NaN must land where the oracle has NaN.
        nan = np.isnan(ref)
        assert_bitwise(got[~nan], ref[~nan], f"directed step={step}")
        assert np.isnan(got[nan]).all()
        assert n * 3 == got.size


def test_optimizer_workload_full_size_sampled():
    # n = 1.2e9: w ~ N(0,0.02), m ~ N(0,1e-4), v = |N(0,1e-6)|, g ~ N(0,1e-3),
    # step 1000.  The element update is independent per element, so the
    # oracle runs on gathered samples (region edges plus random indices).
    cfg = synth.ADAMW
    n = cfg["n"]
    print(f"adamw workload n={n}", flush=True)
    state = torch.empty(3 * n, dtype=torch.float32, device="cuda")
    grad = torch.empty(n, dtype=torch.float32, device="cuda")
    host = np.empty(n, np.float32)
    samples = {}
    rng = np.random.default_rng(6)
    idx = np.unique(np.concatenate([np.arange(0, 4096), np.arange(n - 4096, n),
                                    rng.integers(0, n, 1_000_000)]))
    for k, (fn, dst) in enumerate([(synth.adamw_w, state[:n]), (synth.adamw_m, state[n:2 * n]),
                                   (synth.adamw_v, state[2 * n:]), (synth.adamw_g, grad)]):
        fn(n, out=host)
        dst.copy_(torch.from_numpy(host))
        samples[k] = host[idx].copy()
    del host
    hp = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"], weight_decay=cfg["wd"])
    br.repro_adamw(state, grad, step=cfg["step"], **hp)
    torch.cuda.synchronize()
    tidx = torch.from_numpy(idx).cuda()
    got = [to_host(state[:n][tidx]), to_host(state[n:2 * n][tidx]), to_host(state[2 * n:][tidx])]
    ref = oracle.adamw(np.concatenate([samples[0], samples[1], samples[2]]), samples[3], step=cfg["step"], **hp)
    k = idx.size
    assert_bitwise(got[0], ref[:k], "w")
    assert_bitwise(got[1], ref[k:2 * k], "m")
    assert_bitwise(got[2], ref[2 * k:], "v")


def test_errors():
    lib = br.library()
    d = torch.zeros(12, device="cuda")
    p = d.data_ptr()
    assert lib.repro_adamw(p, p, 4, 1e-3, 0.9, 0.999, 1e-8, 0.1, 0, None) == -1  # step 0
    assert lib.repro_adamw(p + 2, p, 4, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1, None) == -2
