"""GPU parity: the pre-clip gradient norm and the BF16-parameter optimizer
step (clip, spike rule, fused update) against the oracle, bit for bit.

OPEN-1B paper, sections 3.1, 3.2 ("Optimizer", "Optimizer-state precision")
and 3.4.2; Appendix A.1 for the order of the norm's sum.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _grad(n, tid, std):
    return synth.generate(n, synth.OUTLIER_SCALED, tid, std, 0.001, 30.0)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 4095, 4096, 4097, 12_289, 100_003, (1 << 24) + 4099])
@pytest.mark.parametrize("bf16", [False, True])
def test_grad_norm_matches_oracle(n, bf16):
    g = _grad(n, 0xA000 + n % 997, 1e-3)
    if bf16:
        gb = _bf16_bits(g)
        ref_norm, ref_S = oracle.grad_norm(gb, return_sumsq=True)
        out = to_host(br.repro_grad_norm(_dev_bf16(gb)))
    else:
        ref_norm, ref_S = oracle.grad_norm(g, return_sumsq=True)
        out = to_host(br.repro_grad_norm(to_dev(g)))
    assert_bitwise(out, np.array([ref_norm, ref_S], np.float32), f"norm n={n} bf16={bf16}")


def test_grad_norm_unaligned_order_witness_and_empty():
    g = np.ones(4097 * 3, np.float32)
    g[0] = 4096.0
    ref = np.array(oracle.grad_norm(g[1:], return_sumsq=True), np.float32)
    out = to_host(br.repro_grad_norm(to_dev(g)[1:]))  # 4-byte aligned view: scalar loads
    assert_bitwise(out, ref, "unaligned view")
    gb = _bf16_bits(g)
    ref_b = np.array(oracle.grad_norm(gb[3:], return_sumsq=True), np.float32)
    out_b = to_host(br.repro_grad_norm(_dev_bf16(gb)[3:]))  # 2-byte aligned bf16 view
    assert_bitwise(out_b, ref_b, "unaligned bf16 view")
    w = np.ones(4096, np.float32)
    w[0] = 4096.0
    out = to_host(br.repro_grad_norm(to_dev(w)))
    assert out[1] == np.float32(2.0 ** 24 + 4094)
    out = to_host(br.repro_grad_norm(torch.zeros(0, device="cuda")))
    assert (out == 0).all()


def _state_dict(st):
    return {k: st[k][0].item() for k in st.dtype.names}


def _run_steps(n, gs, bf16_grad, seed, max_norm=1.0, spike=5.0, skip=5, views=False):
    rng = np.random.default_rng(seed)
    w = _bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    if views:  # 2- and 4-byte aligned views take the scalar update kernel
        dw = _dev_bf16(np.concatenate([[0], w]).astype(np.uint16))[1:]
        dm = to_dev(np.concatenate([[0], m]).astype(np.float32))[1:]
        dv = to_dev(np.concatenate([[0], v]).astype(np.float32))[1:]
    else:
        dw, dm, dv = _dev_bf16(w), to_dev(m), to_dev(v)
    st_dev = br.new_step_state()
    st_ref = oracle.new_step_state()
    ws = br.grad_norm_workspace(n)
    for k, g in enumerate(gs):
        gin = _bf16_bits(g) if bf16_grad else g
        dg = _dev_bf16(gin) if bf16_grad else to_dev(gin)
        br.repro_adamw_bf16_step(dw, dm, dv, dg, st_dev, **HP, max_norm=max_norm, spike_threshold=spike,
                                 skip_steps=skip, workspace=ws)
        oracle.adamw_bf16_step(w, m, v, gin, st_ref, **HP, max_norm=max_norm, spike_threshold=spike,
                               skip_steps=skip)
        what = f"n={n} step {k} bf16_grad={bf16_grad}"
        assert np.array_equal(_host_bits(dw), w), what + " w"
        assert_bitwise(to_host(dm), m, what + " m")
        assert_bitwise(to_host(dv), v, what + " v")
        got = br.read_step_state(st_dev)
        ref = _state_dict(st_ref)
        for key in ("step", "skip_left", "applied"):
            assert got[key] == ref[key], (what, key, got, ref)
        for key in ("grad_norm", "clip_coef", "beta1_pow", "beta2_pow"):
            assert np.float32(got[key]).view(np.uint32) == np.float32(ref[key]).view(np.uint32), (what, key)
    return _state_dict(st_ref)


@pytest.mark.parametrize("n", [1, 5, 4096, 10_007, 300_001])
@pytest.mark.parametrize("bf16_grad", [False, True])
def test_step_sequence_with_clip_and_spike(n, bf16_grad):
    # Gradient scales chosen so that the norm stays below 1, lands between 1
    # and 5 (clipped), and exceeds 5 (skipped), whatever n is.
    def g_of(k, target):
        x = _grad(n, 0xA100 + 16 * k + n % 13, 1.0)
        nrm = float(np.sqrt(np.sum(x.astype(np.float64) ** 2)))
        return (x * np.float32(target / nrm)).astype(np.float32)
    targets = [0.5, 3.0, 7.0, 0.5, 2.0, 0.5, 0.5, 0.5, 4.0, 0.2]
    ref = _run_steps(n, [g_of(k, t) for k, t in enumerate(targets)], bf16_grad, n)
    assert ref["step"] == 5  # the spike at step 2 skipped steps 2..6


def test_views_and_no_rule():
    n = 9_999
    gs = [_grad(n, 0xA200 + k, 1e-3) for k in range(3)]
    _run_steps(n, gs, False, 1, views=True)
    _run_steps(n, gs, True, 2, max_norm=0.0, spike=0.0)


def test_full_size_step_sampled():
    # The optimizer workload of the recipe: n = 1.2e9 bf16 parameters, FP32
    # moments, a bf16 gradient whose norm (~3.5) is clipped to 1.
    n = synth.ADAMW["n"]
    print(f"bf16 step n={n}", flush=True)
    rng = np.random.default_rng(21)
    idx = np.unique(np.concatenate([np.arange(0, 2048), np.arange(n - 2048, n), rng.integers(0, n, 40_000)]))
    g32 = synth.generate(n, synth.NORMAL, synth.tid(7, 3), 1e-4)
    gb = _bf16_bits(g32)
    del g32
    ref_norm, _ = oracle.grad_norm(gb, return_sumsq=True)
    w = _bf16_bits(synth.adamw_w())
    m = synth.adamw_m()
    v = synth.adamw_v()
    ws, ms, vs, gs = w[idx].copy(), m[idx].copy(), v[idx].copy(), gb[idx].copy()
    dw, dm, dv, dg = _dev_bf16(w), to_dev(m), to_dev(v), _dev_bf16(gb)
    del w, m, v, gb
    st = br.new_step_state()
    br.repro_adamw_bf16_step(dw, dm, dv, dg, st, **HP)
    got = br.read_step_state(st)
    assert np.float32(got["grad_norm"]) == ref_norm and got["applied"] == 1
    coef = np.float32(1.0) / (ref_norm + np.float32(1e-6))
    assert coef < 1 and np.float32(got["clip_coef"]) == coef
    # The sampled elements through the oracle with the same coefficient
    # applied first (one binary32 product, as the step does) and no rule.
    gc = (oracle.bf16_widen(gs) * coef).astype(np.float32)
    so = oracle.new_step_state()
    oracle.adamw_bf16_step(ws, ms, vs, gc, so, **HP, max_norm=0.0, spike_threshold=0.0)
    tidx = torch.from_numpy(idx).cuda()
    assert np.array_equal(_host_bits(dw[tidx]), ws)
    assert_bitwise(to_host(dm[tidx]), ms, "full-size m")
    assert_bitwise(to_host(dv[tidx]), vs, "full-size v")


def test_errors():
    lib = br.library()
    d = torch.zeros(1024, device="cuda")
    p = d.data_ptr()
    ws = br.grad_norm_workspace(100)
    assert lib.repro_grad_norm(p, 2, 100, ws.data_ptr(), ws.numel(), p, None) == -1   # bad dtype
    assert lib.repro_grad_norm(p, 0, 100, ws.data_ptr(), 16, p, None) == -4          # workspace too small
    assert lib.repro_grad_norm(p, 0, 100, ws.data_ptr() + 16, ws.numel(), p, None) == -2
    assert lib.repro_grad_norm(p + 2, 0, 100, ws.data_ptr(), ws.numel(), p, None) == -2
    assert lib.repro_adamw_bf16_step(p, p, p, p, 0, 100, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 5.0, -1, ws.data_ptr(),
                                     ws.numel(), p, None) == -1  # negative skip_steps
    assert lib.repro_adamw_bf16_step(p, p, p, p, 0, 100, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0, 5.0, 5, ws.data_ptr(),
                                     ws.numel(), p + 4, None) == -2  # state not 8-byte aligned
