"""Pins for the oracle's BF16-parameter optimizer step (CPU only).

OPEN-1B paper: section 3.1 (parameters held in BF16, FP32 gradient
reduction), section 3.2 "Optimizer" (AdamW; gradients clipped to a global
l2 norm of 1.0) and "Optimizer-state precision" (the fused step widens BF16
parameter and gradient to FP32, updates in FP32 with FP32 moments, rounds the
parameter to BF16 once), section 3.4.2 (five optimizer steps skipped when the
pre-clip norm exceeds 5).

Independent references: torch's float32 <-> bfloat16 conversions (IEEE
round-to-nearest-even), the pinned FP32 AdamW oracle, the pinned vector
TreeFold, and exact integer sums.
"""
import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _torch_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * 2.0 ** rng.integers(-125, 120, 200_000)).astype(np.float32)
    # Exact ties (the 16 dropped bits are 0x8000) on both parities, and values
    # next to the smallest normal.
    t = rng.integers(0, 2 ** 31, 10_000).astype(np.uint32) & np.uint32(0xFFFF0000) | np.uint32(0x8000)
    t = t[(((t >> 23) & 0xFF) > 0) & (((t >> 23) & 0xFF) < 0xFF)]  # finite normals
    edge = np.array([2.0 ** -126, -(2.0 ** -126), 2.0 ** -126 * (1 + 2.0 ** -9), 0.0, -0.0, 1.0, 3.0e38,
                     3.3895e38, -3.3895e38, 3.3961e38, -3.3961e38, 3.4028e38], np.float32)
    for arr in (x, t.view(np.float32), edge):
        np.testing.assert_array_equal(oracle.bf16_round(arr), _torch_bf16(arr))


def test_bf16_widen_matches_torch():
    h = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16)
    h = h[((h >> 7) & 0xFF) != 0xFF]  # finite patterns
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(_bits(oracle.bf16_widen(h)), _bits(ref))


def _norm_via_tree(g):
    q = (np.asarray(g, np.float32) * np.asarray(g, np.float32)).astype(np.float32)
    S = oracle.tree_reduce([q[i:i + 1] for i in range(q.size)], average=False)[0]
    return np.float32(np.sqrt(np.float64(S)))  # a binary64 sqrt rounds to the correct binary32 sqrt


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 8, 13, 31, 64])
def test_grad_norm_is_the_treefold_of_squares(n):
    rng = np.random.default_rng(n)
    g = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    assert oracle.grad_norm(g) == _norm_via_tree(g)


def test_grad_norm_order_witness():
    # g = [4096, 1 x 4095]: the fold adds the ones in pairs before they meet
    # 2^24 and keeps them (S = 2^24 + 4094); a left-to-right sum loses each
    # one against 2^24 (S = 2^24).
    g = np.ones(4096, np.float32)
    g[0] = 4096
    assert oracle.grad_norm(g) == np.float32(np.sqrt(2.0 ** 24 + 4094))
    assert oracle.grad_norm(g) != np.float32(4096)


def test_fold_result_starts_from_the_smallest_block():
    # n = 7: blocks (q0..q3), (q4, q5), (q6).  Squares [2^24, 0, 0, 0, 1, 0, 1]:
    # Result = (q6 + (q4 + q5)) + block0 = 2 + 2^24, exact.  Starting from the
    # largest block, (2^24 + 1) + 1 loses both ones.
    g = np.array([4096, 0, 0, 0, 1, 0, 1], np.float32)
    _, S = oracle.grad_norm(g, return_sumsq=True)
    assert S == np.float32(2.0 ** 24 + 2)


def test_grad_norm_exact_integer_case_and_bf16_input():
    rng = np.random.default_rng(3)
    g = rng.integers(-3, 4, 100_001).astype(np.float32)
    S = int(np.sum(g.astype(np.int64) ** 2))
    assert S < 2 ** 24
    want = np.float32(np.sqrt(np.float64(S)))
    assert oracle.grad_norm(g) == want
    assert oracle.grad_norm(_torch_bf16(g)) == want  # small integers are exact in bf16
    assert oracle.grad_norm(np.zeros(0, np.float32)) == 0


def _fresh(n, seed, g_dtype="f32"):
    rng = np.random.default_rng(seed)
    w = _torch_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    return w, m, v


def _reference_step(w, m, v, g, t):
    """The FP32 oracle step on the widened parameter, then torch's bf16 rounding."""
    n = w.size
    st = np.concatenate([oracle.bf16_widen(w), m, v]).astype(np.float32)
    oracle.adamw_inplace(st, np.asarray(g, np.float32), HP["lr"], HP["beta1"], HP["beta2"], HP["eps"],
                         HP["weight_decay"], t)
    return _torch_bf16(st[:n]), st[n:2 * n].copy(), st[2 * n:].copy()


def test_unclipped_steps_equal_the_fp32_update_rounded_once():
    n = 5000
    w, m, v = _fresh(n, 1)
    ws, ms, vs = w.copy(), m.copy(), v.copy()
    state = oracle.new_step_state()
    rng = np.random.default_rng(2)
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        oracle.adamw_bf16_step(w, m, v, g, state, **HP, max_norm=0.0, spike_threshold=0.0)
        ws, ms, vs = _reference_step(ws, ms, vs, g, t)
        np.testing.assert_array_equal(w, ws)
        np.testing.assert_array_equal(_bits(m), _bits(ms))
        np.testing.assert_array_equal(_bits(v), _bits(vs))
        assert state["step"][0] == t and state["applied"][0] == 1
        p1 = np.float32(HP["beta1"])
        for _ in range(t - 1):
            p1 = np.float32(p1 * np.float32(HP["beta1"]))
        assert state["beta1_pow"][0] == p1


def test_bf16_gradient_is_widened_exactly():
    n = 3000
    w, m, v = _fresh(n, 4)
    gh = _torch_bf16((np.random.default_rng(5).standard_normal(n) * 1e-3).astype(np.float32))
    w2, m2, v2 = w.copy(), m.copy(), v.copy()
    oracle.adamw_bf16_step(w, m, v, gh, oracle.new_step_state(), **HP, max_norm=0.0, spike_threshold=0.0)
    oracle.adamw_bf16_step(w2, m2, v2, oracle.bf16_widen(gh), oracle.new_step_state(), **HP, max_norm=0.0,
                           spike_threshold=0.0)
    np.testing.assert_array_equal(w, w2)
    np.testing.assert_array_equal(_bits(m), _bits(m2))


@pytest.mark.parametrize("scale", [1.0, 0.0205])
def test_clip_scales_every_element_by_the_coefficient(scale):
    # Norms ~63 and ~1.3 (where the 1e-6 of the denominator moves the
    # coefficient by several ulps).
    n = 4000
    w, m, v = _fresh(n, 6)
    g = (np.random.default_rng(7).standard_normal(n) * scale).astype(np.float32)
    norm = _norm_via_tree(g)
    coef = np.float32(1.0) / (norm + np.float32(1e-6))
    assert coef < 1
    assert scale == 1.0 or coef != np.float32(1.0) / norm
    gc = (g * coef).astype(np.float32)
    ws, ms, vs = _reference_step(w, m, v, gc, 1)
    state = oracle.new_step_state()
    oracle.adamw_bf16_step(w, m, v, g, state, **HP, max_norm=1.0, spike_threshold=0.0)
    assert state["grad_norm"][0] == norm and state["clip_coef"][0] == coef
    np.testing.assert_array_equal(w, ws)
    np.testing.assert_array_equal(_bits(m), _bits(ms))
    # Below the threshold nothing is scaled.
    w, m, v = _fresh(n, 6)
    small = (g * np.float32(1e-3)).astype(np.float32)
    ws, ms, vs = _reference_step(w, m, v, small, 1)
    state = oracle.new_step_state()
    oracle.adamw_bf16_step(w, m, v, small, state, **HP, max_norm=1.0, spike_threshold=0.0)
    assert state["clip_coef"][0] == 1
    np.testing.assert_array_equal(_bits(m), _bits(ms))


def test_spike_protocol_skips_five_steps_without_advancing_the_count():
    n = 2000
    w, m, v = _fresh(n, 8)
    rng = np.random.default_rng(9)
    base = (rng.standard_normal(n) * 1e-3).astype(np.float32)   # norm ~ 0.045
    spike = (rng.standard_normal(n) * 0.2).astype(np.float32)   # norm ~ 9 > 5
    state = oracle.new_step_state()
    # Step pattern: apply, spike (skip), 4 more skipped, apply.
    seq = [base, spike, base, base, base, base, base]
    applied = []
    ws, ms, vs = w.copy(), m.copy(), v.copy()
    t = 0
    for g in seq:
        before = w.copy()
        oracle.adamw_bf16_step(w, m, v, g, state, **HP, max_norm=1.0, spike_threshold=5.0, skip_steps=5)
        applied.append(int(state["applied"][0]))
        if applied[-1]:
            t += 1
            coef = min(np.float32(1), np.float32(1) / (_norm_via_tree(g) + np.float32(1e-6)))
            gc = g if coef == 1 else (g * coef).astype(np.float32)
            ws, ms, vs = _reference_step(ws, ms, vs, gc, t)
            np.testing.assert_array_equal(w, ws)
            np.testing.assert_array_equal(_bits(v), _bits(vs))
        else:
            np.testing.assert_array_equal(w, before)
    assert applied == [1, 0, 0, 0, 0, 0, 1]
    assert state["step"][0] == 2 and state["skip_left"][0] == 0


def test_spike_inside_the_window_starts_it_again():
    n = 500
    w, m, v = _fresh(n, 10)
    rng = np.random.default_rng(11)
    base = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    spike = (rng.standard_normal(n) * 0.5).astype(np.float32)
    state = oracle.new_step_state()
    pattern = []
    for g in [spike, base, spike, base, base, base, base, base]:
        oracle.adamw_bf16_step(w, m, v, g, state, **HP, max_norm=1.0, spike_threshold=5.0, skip_steps=5)
        pattern.append(int(state["applied"][0]))
    assert pattern == [0, 0, 0, 0, 0, 0, 0, 1]
    assert state["step"][0] == 1
