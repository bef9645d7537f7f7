"""Pins for the oracle AdamW step (CPU only).

OPEN-1B paper, section 3.2 "Optimizer" (AdamW of Loshchilov and Hutter with
decoupled weight decay, through a fused reproducible kernel) and
"Optimizer-state precision" (FP32 moments); the checkpoint page's file format
(flat [w | m | v], beta1 = 0.9, beta2 = 0.999); Appendix A.3 (tensor / scalar
realised as a multiply by a host-computed reciprocal, here applied to the bias
corrections).

Element update, with m_hat = m' * r1, v_hat = v' * r2:
    m' = beta1 m + (1-beta1) g,  v' = beta2 v + (1-beta2) g^2,
    w' = w - lr (m_hat / (sqrt(v_hat) + eps) + wd w).
"""
import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -24


def _state(w, m, v):
    return np.concatenate([w, m, v]).astype(np.float32)


def test_dyadic_case_is_exact():
    # beta1 = 1/2, beta2 = 3/4, eps = 0, lr = 2^-4, wd = 2^-2, step 1,
    # m = v = 0: c1 = 1/2, c2 = 1/4, bc1 = 1/2, bc2 = 1/4, r1 = 2, r2 = 4,
    # so m_hat = g, v_hat = g^2, sqrt exact, u = sign(g), and
    # w' = w - (sign(g) + w/4)/16, all exact for small integers.
    rng = np.random.default_rng(0)
    n = 1000
    w = rng.integers(-64, 65, n).astype(np.float32)
    g = rng.integers(1, 50, n).astype(np.float32) * rng.choice([-1.0, 1.0], n).astype(np.float32)
    st = oracle.adamw(_state(w, np.zeros(n), np.zeros(n)), g, lr=2.0 ** -4, beta1=0.5, beta2=0.75,
                      eps=0.0, weight_decay=0.25, step=1)
    w_exp = w.astype(np.float64) - (np.sign(g) + w / 4.0) / 16.0
    np.testing.assert_array_equal(st[:n].astype(np.float64), w_exp)
    np.testing.assert_array_equal(st[n:2 * n].astype(np.float64), g.astype(np.float64) / 2)
    np.testing.assert_array_equal(st[2 * n:].astype(np.float64), g.astype(np.float64) ** 2 / 4)


def test_host_scalars():
    c1, c2, r1, r2 = oracle.adamw_scalars(0.9, 0.999, 1)
    # 1 - 0.9f is exact (Sterbenz); r1 = fl(1 / c1).
    assert c1 == np.float32(1) - np.float32(0.9)
    assert c2 == np.float32(1) - np.float32(0.999)
    assert r1 == np.float32(1) / c1 and r2 == np.float32(1) / c2
    # At step 1000 the serial product 0.9^t drops below 2^-126 (from about
    # t = 829 on) and is flushed, so bc1 = 1 and r1 = 1 exactly; 0.999^1000
    # stays normal: r2 ~ 1/(1 - 0.999^1000) within the rounding of 999
    # serial binary32 products.
    c1, c2, r1, r2 = oracle.adamw_scalars(0.9, 0.999, 1000)
    assert r1 == 1.0
    b2 = np.float64(np.float32(0.999))
    assert abs(r2 / (1.0 / (1.0 - b2 ** 1000)) - 1) < 1e-4
    with pytest.raises(ValueError):
        oracle.adamw_scalars(0.9, 0.999, 0)


def test_first_step_closed_form():
    # From m = v = 0 at step 1: m_hat = g and v_hat = g^2 in exact
    # arithmetic, so w' = w - lr (g / (|g| + eps) + wd w).  The binary32 chain
    # has 16 roundings; a first-order bound on the error of w' is
    # u (|w'| + 2|t| + 10 lr |u_exact|) with t = lr (u + wd w).
    rng = np.random.default_rng(1)
    n = 100_000
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    lr, wd, eps = 1e-3, 0.1, 1e-8
    st = oracle.adamw(_state(w, np.zeros(n), np.zeros(n)), g, lr, 0.9, 0.999, eps, wd, 1)
    w64, g64 = w.astype(np.float64), g.astype(np.float64)
    lr64, wd64, eps64 = (np.float64(np.float32(x)) for x in (lr, wd, eps))
    u_ex = g64 / (np.abs(g64) + eps64)
    t_ex = lr64 * (u_ex + wd64 * w64)
    w_ex = w64 - t_ex
    bound = U * (np.abs(w_ex) + 2 * np.abs(t_ex) + 10 * lr64 * np.abs(u_ex)) + 1e-30
    assert (np.abs(st[:n] - w_ex) <= bound).all()
    # eps really sits outside the root: with |g| ~ eps the alternative
    # g / sqrt(g^2 + eps) would be far away.
    assert np.abs(u_ex).max() < 1.0


def test_constant_gradient_trajectory():
    # With a constant gradient g, m_hat_t = g and v_hat_t = g^2 at every t in
    # exact arithmetic (the bias corrections cancel the (1 - beta^t)
    # factors), so w_t = w_{t-1} - lr (g / (|g| + eps) + wd w_{t-1}).
    # A wrong bias correction, a swapped moment or eps under the root breaks
    # this by far more than the accumulated rounding.
    rng = np.random.default_rng(2)
    n = 20_000
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    lr, wd, eps = 3e-4, 0.1, 1e-8
    st = _state(w, np.zeros(n), np.zeros(n))
    w64 = w.astype(np.float64)
    g64 = g.astype(np.float64)
    lr64, wd64, eps64 = (np.float64(np.float32(x)) for x in (lr, wd, eps))
    for t in range(1, 41):
        st = oracle.adamw(st, g, lr, 0.9, 0.999, eps, wd, t)
        w64 = w64 - lr64 * (g64 / (np.abs(g64) + eps64) + wd64 * w64)
        # The moment ratios drift from exact by ~40 roundings per step.
        tol = 200 * t * U * (np.abs(w64) + lr64)
        assert (np.abs(st[:n] - w64) <= tol).all(), t


def test_matches_torch_adamw_in_float64():
    # torch.optim.AdamW computes the same update in another algebraic form
    # (w (1 - lr wd), then lr/bc1 * m / (sqrt(v)/sqrt(bc2) + eps)).  Run in
    # float64 it is the exact-arithmetic reference within ~1e-15; the oracle
    # must agree within binary32 rounding over several steps.
    rng = np.random.default_rng(3)
    n = 50_000
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    lr, b1, b2, eps, wd = 3e-4, 0.9, 0.999, 1e-8, 0.1
    f32 = lambda x: float(np.float32(x))
    p = torch.nn.Parameter(torch.tensor(w, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=f32(lr), betas=(f32(b1), f32(b2)), eps=f32(eps), weight_decay=f32(wd))
    # Start torch from the same moments at step 10: seed its state directly.
    start = 10
    opt.state[p] = {"step": torch.tensor(float(start - 1), dtype=torch.float64),
                    "exp_avg": torch.tensor(m, dtype=torch.float64),
                    "exp_avg_sq": torch.tensor(v, dtype=torch.float64)}
    st = _state(w, m, v)
    for t in range(start, start + 5):
        gt = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        p.grad = torch.tensor(gt, dtype=torch.float64)
        opt.step()
        st = oracle.adamw(st, gt, lr, b1, b2, eps, wd, t)
    ref_w = p.detach().numpy()
    ref_m = opt.state[p]["exp_avg"].numpy()
    ref_v = opt.state[p]["exp_avg_sq"].numpy()
    # Each step rounds w' (half an ulp of |w|) and carries ~20 roundings of
    # relative size u on the step lr (u + wd w), |u| <= ~3.
    assert (np.abs(st[:n] - ref_w) <= 5 * U * (np.abs(ref_w) + 60 * lr)).all()
    # Moments: each step adds at most ~1.5 u (|beta m| + |(1-beta) g|) of
    # rounding, and the errors decay geometrically; 20 u of the largest
    # magnitude covers five steps.
    assert np.abs(st[n:2 * n] - ref_m).max() <= 20 * U * np.abs(ref_m).max()
    assert np.abs(st[2 * n:] - ref_v).max() <= 20 * U * np.abs(ref_v).max()
    # The weight change itself (~3e-5 against |w| ~ 0.02, so its relative
    # error is dominated by the rounding of w') agrees to ~1e-4.
    dw_o = st[:n].astype(np.float64) - w
    dw_t = ref_w - w
    assert np.median(np.abs(dw_o - dw_t) / np.abs(dw_t)) < 1e-4


def test_other_algebraic_forms_change_bits():
    # Non-vacuity: the torch-style folding evaluated in binary32 (w * (1 -
    # lr wd), division by the bias corrections) lands on different bits for
    # some elements, so parity tests on this data can tell the declared
    # sequence from an equivalent-looking one.
    rng = np.random.default_rng(4)
    n = 100_000
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    lr, b1, b2, eps, wd, t = (np.float32(x) for x in (3e-4, 0.9, 0.999, 1e-8, 0.1, 7))
    st = oracle.adamw(_state(w, m, v), g, lr, b1, b2, eps, wd, 7)
    one = np.float32(1)
    mn = b1 * m + (one - b1) * g
    vn = b2 * v + (one - b2) * (g * g)
    bc1 = one - b1 ** np.float32(7)
    bc2 = one - b2 ** np.float32(7)
    alt = w * (one - lr * wd) - (lr / bc1) * mn / (np.sqrt(vn) / np.sqrt(bc2) + eps)
    assert (alt.astype(np.float32) != st[:n]).sum() > 100


def test_empty_and_bad_step():
    assert oracle.adamw(np.zeros(0, np.float32), np.zeros(0, np.float32), 1e-3, 0.9, 0.999, 1e-8, 0.1, 1).size == 0
    with pytest.raises(ValueError):
        oracle.adamw(np.zeros(3, np.float32), np.zeros(1, np.float32), 1e-3, 0.9, 0.999, 1e-8, 0.1, 0)
