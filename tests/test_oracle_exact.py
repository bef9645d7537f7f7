"""The oracle against exact rational arithmetic (CPU only).

`exact_fp32` computes each binary32 operation from its definition (the exact
result as a fraction, one rounding to nearest-even at 24 bits, then the
contract's flush rule; OPEN-1B section 2.1 and Table 1).  Every primitive
operation of the oracle, and its GEMM chain, TreeFold and AdamW element
sequence built from them, must equal that word for word on random operands
across the exponent range and on sets built around the flush boundary,
overflow, ties and cancellation.  This pins the oracle's arithmetic to the
definitions independently of the host's floating-point unit.
"""
import numpy as np
import pytest

import exact_fp32 as X
import oracle

OPS = {oracle.OP_ADD: X.add, oracle.OP_SUB: X.sub, oracle.OP_MUL: X.mul, oracle.OP_DIV: X.div,
       oracle.OP_SQRT: lambda a, b: X.sqrt(a)}


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _words(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _operands(op, seed, n=3000):
    rng = np.random.default_rng(seed)
    sign = lambda k: rng.choice([-1.0, 1.0], k)  # noqa: E731
    k = n // 6
    sets = []
    # Random exponents over the whole range (some operands subnormal or tiny).
    sets.append((rng.uniform(1, 2, k) * 2.0 ** rng.integers(-140, 120, k) * sign(k),
                 rng.uniform(1, 2, k) * 2.0 ** rng.integers(-140, 120, k) * sign(k)))
    # Results at the flush boundary: products and quotients near 2^-126.
    m = (1 + rng.integers(-6, 7, k) * 2.0 ** -23)
    sets.append((m * 2.0 ** -63 * sign(k), (1 + rng.integers(-6, 7, k) * 2.0 ** -23) * 2.0 ** -63 * sign(k)))
    # Sums and differences near 2^-126 (exact in binary32 arithmetic, then flushed or not).
    sets.append((rng.uniform(1, 2, k) * 2.0 ** -126 * sign(k), rng.uniform(1, 2, k) * 2.0 ** -126 * sign(k)))
    # Exact ties for addition and multiplication.
    i = 2 * rng.integers(0, 2000, k) + 1
    sets.append(((1 + i * 2.0 ** -12) * sign(k), (1 + (2 * rng.integers(0, 2000, k) + 1) * 2.0 ** -12)))
    # Cancellation: b close to -a.
    a = rng.uniform(1, 2, k) * 2.0 ** rng.integers(-100, 100, k) * sign(k)
    sets.append((a, -a * (1 + rng.integers(-3, 4, k) * 2.0 ** -22)))
    # Near overflow.
    sets.append((rng.uniform(1, 2, k) * 2.0 ** rng.integers(60, 127, k) * sign(k),
                 rng.uniform(1, 2, k) * 2.0 ** rng.integers(0, 70, k) * sign(k)))
    a = _f32(np.concatenate([s[0] for s in sets]))
    b = _f32(np.concatenate([s[1] for s in sets]))
    if op == oracle.OP_SQRT:
        a = np.abs(a)
    if op == oracle.OP_DIV:
        b = np.where(np.abs(b) < 2.0 ** -126, np.float32(1.5), b).astype(np.float32)  # nonzero divisors
    # Signed zeros and subnormals against each other and against normals.
    z = _f32([0.0, -0.0, 2.0 ** -140, -(2.0 ** -149), 2.0 ** -126, -(2.0 ** -126), 1.0, -3.0])
    za, zb = np.meshgrid(z, z)
    za, zb = za.reshape(-1), zb.reshape(-1)
    if op == oracle.OP_SQRT:
        za = np.abs(za)
    if op == oracle.OP_DIV:
        keep = np.abs(zb) >= 2.0 ** -126
        za, zb = za[keep], zb[keep]
    return np.concatenate([a, za]).astype(np.float32), np.concatenate([b, zb]).astype(np.float32)


@pytest.mark.parametrize("op", list(OPS))
def test_primitive_operations(op):
    a, b = _operands(op, 700 + op)
    got = oracle.fp32_op(op, a, b)
    want = np.array([OPS[op](x, y) for x, y in zip(a, b)], np.float32)
    bad = np.nonzero(_words(got) != _words(want))[0]
    assert bad.size == 0, [(float(a[i]), float(b[i]), float(got[i]), float(want[i])) for i in bad[:5]]
    # The sets reach both sides of the flush boundary and overflow where they can.
    if op in (oracle.OP_MUL, oracle.OP_ADD, oracle.OP_SUB):
        assert (want == 0).sum() > 50 and (np.abs(want) == np.float32(2.0 ** -126)).sum() > 0
    if op == oracle.OP_MUL:
        assert np.isinf(want).sum() > 10


def _chain(A, B):
    M, K = A.shape
    N = B.shape[1]
    C = np.zeros((M, N), np.float32)
    for i in range(M):
        for j in range(N):
            acc = np.float32(0.0)
            for k in range(K):
                acc = X.add(acc, X.mul(A[i, k], B[k, j]))
            C[i, j] = acc
    return C


def test_gemm_chain():
    rng = np.random.default_rng(9)
    for M, N, K in ((3, 4, 9), (5, 2, 17)):
        A = _f32(rng.uniform(1, 2, (M, K)) * 2.0 ** rng.integers(-70, 20, (M, K)) * rng.choice([-1, 1], (M, K)))
        B = _f32(rng.uniform(1, 2, (K, N)) * 2.0 ** rng.integers(-70, 20, (K, N)) * rng.choice([-1, 1], (K, N)))
        A[0, :3] = _f32([2.0 ** -63, -(2.0 ** -64), 2.0 ** -140])
        ref = _chain(A, B)
        assert np.array_equal(_words(oracle.gemm(A, B)), _words(ref)), (M, N, K)
        assert np.array_equal(_words(oracle.gemm(np.ascontiguousarray(A.T), B, trans_a=True)), _words(ref))


def _treefold(xs):
    """Push / Result of Appendix A.1's Algorithm 2, written on exact operations."""
    stack = []
    for x in xs:
        level = 0
        while stack and stack[-1][0] == level:
            x = X.add(stack.pop()[1], x)
            level += 1
        stack.append((level, x))
    acc = stack[-1][1]  # the lowest level, then the others in ascending level
    for _, part in reversed(stack[:-1]):
        acc = X.add(acc, part)
    return acc


@pytest.mark.parametrize("R", [3, 7, 8, 13])
def test_tree_reduce(R):
    rng = np.random.default_rng(100 + R)
    n = 40
    reps = [_f32(rng.standard_normal(n) * 10.0 ** rng.integers(-3, 4, n)) for _ in range(R)]
    reps[0][:4] = _f32([2.0 ** -126, -(2.0 ** -126), 1.5 * 2.0 ** -126, 2.0 ** 24])
    rR = X.div(np.float32(1.0), np.float32(R))
    want = np.array([X.mul(_treefold([r[i] for r in reps]), rR) for i in range(n)], np.float32)
    assert np.array_equal(_words(oracle.tree_reduce(reps)), _words(want))
    plain = np.array([_treefold([r[i] for r in reps]) for i in range(n)], np.float32)
    assert np.array_equal(_words(oracle.tree_reduce(reps, average=False)), _words(plain))


def _adamw_exact(w, m, v, g, lr, b1, b2, eps, wd, step):
    lr, b1, b2, eps, wd = (np.float32(x) for x in (lr, b1, b2, eps, wd))
    one = np.float32(1.0)
    c1, c2 = X.sub(one, b1), X.sub(one, b2)
    p1, p2 = b1, b2
    for _ in range(2, step + 1):
        p1, p2 = X.mul(p1, b1), X.mul(p2, b2)
    r1 = X.div(one, X.sub(one, p1))
    r2 = X.div(one, X.sub(one, p2))
    out = []
    for wi, mi, vi, gi in zip(w, m, v, g):
        mn = X.add(X.mul(b1, mi), X.mul(c1, gi))
        vn = X.add(X.mul(b2, vi), X.mul(c2, X.mul(gi, gi)))
        u = X.div(X.mul(mn, r1), X.add(X.sqrt(X.mul(vn, r2)), eps))
        wn = X.sub(wi, X.mul(lr, X.add(u, X.mul(wd, wi))))
        out.append((wn, mn, vn))
    return [np.array(c, np.float32) for c in zip(*out)]


@pytest.mark.parametrize("step", [1, 2, 829, 830, 1000])
def test_adamw_element_sequence(step):
    rng = np.random.default_rng(50 + step)
    n = 64
    w = _f32(rng.standard_normal(n) * 0.02)
    m = _f32(rng.standard_normal(n) * 1e-4)
    v = _f32(np.abs(rng.standard_normal(n)) * 1e-6)
    g = _f32(rng.standard_normal(n) * 1e-3)
    g[:3] = _f32([0.0, 2.0 ** -70, -(2.0 ** -60)])  # squares that flush
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=step)
    got = oracle.adamw(np.concatenate([w, m, v]), g, **hp)
    wn, mn, vn = _adamw_exact(w, m, v, g, 3e-4, 0.9, 0.999, 1e-8, 0.1, step)
    assert np.array_equal(_words(got), _words(np.concatenate([wn, mn, vn])))


@pytest.mark.parametrize("layout", [(2, 3, 2), (3, 2, 1), (1, 1, 4), (5, 1, 1), (1, 4, 3)])
def test_replay_reduce(layout):
    # Algorithm 1 (section 6) with Appendix A.1-A.3, written on exact operations:
    # microbatch terms scaled before they are added, shards summed in ascending
    # order from a copy of shard 0, each replica's sum scaled and pushed into
    # TreeFold, the result scaled by the replica reciprocal.
    rep_n, shard_n, accum = layout
    rng = np.random.default_rng(sum(layout) * 7 + accum)
    n = 12
    grads = [_f32(rng.standard_normal(n) * 10.0 ** rng.integers(-3, 3, n)) for _ in range(rep_n * shard_n * accum)]
    one = np.float32(1.0)
    ra, rs, rr = (X.div(one, np.float32(d)) for d in (accum, shard_n, rep_n))
    want = np.empty(n, np.float32)
    for i in range(n):
        parts = []
        for rep in range(rep_n):
            inner = None
            for shard in range(shard_n):
                r = rep * shard_n + shard
                g = np.float32(0.0)
                for k in range(accum):
                    g = X.add(g, X.mul(grads[r * accum + k][i], ra))
                inner = g if shard == 0 else X.add(inner, g)
            parts.append(X.mul(inner, rs))
        want[i] = X.mul(_treefold(parts), rr)
    assert np.array_equal(_words(oracle.replay_reduce(grads, *layout)), _words(want))


def _bf16_round_exact(x):
    """binary32 -> bf16 pattern: the exact value rounded to 8 significant bits,
    nearest-even; past the largest bf16, an infinity."""
    s, m = X.decode(x)
    if m == 0:
        return np.uint16(s << 15)
    e = m.numerator.bit_length() - m.denominator.bit_length()
    if X.Fraction(2) ** e > m:
        e -= 1
    q = m / X.Fraction(2) ** (e - 7)
    k = q.numerator // q.denominator
    rem = q - k
    if rem > X.Fraction(1, 2) or (rem == X.Fraction(1, 2) and k % 2 == 1):
        k += 1
    if k == 256:
        k, e = 128, e + 1
    if e > 127:
        return np.uint16((s << 15) | 0x7F80)
    return np.uint16((s << 15) | ((e + 127) << 7) | (k & 0x7F))


def test_bf16_rounding_and_one_clipped_step():
    rng = np.random.default_rng(77)
    n = 96
    x = _f32(rng.uniform(1, 2, 400) * 2.0 ** rng.integers(-120, 127, 400) * rng.choice([-1, 1], 400))
    x[:4] = _f32([3.3895314e38, -3.3961776e38, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])  # overflow and both tie parities
    assert np.array_equal(oracle.bf16_round(x), np.array([_bf16_round_exact(v) for v in x], np.uint16))
    # One BF16 step from m = v = 0 with a gradient whose norm (~3) is clipped to 1.
    w16 = oracle.bf16_round(_f32(rng.standard_normal(n) * 0.02))
    g16 = oracle.bf16_round(_f32(rng.standard_normal(n) * 0.3))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    gw = oracle.bf16_widen(g16)
    S = _treefold([X.mul(gi, gi) for gi in gw])
    norm = X.sqrt(S)
    assert oracle.grad_norm(g16, return_sumsq=True) == (norm, S)
    coef = X.div(np.float32(1.0), X.add(norm, np.float32(1e-6)))
    assert coef < 1
    gc = np.array([X.mul(gi, coef) for gi in gw], np.float32)
    wn, mn, vn = _adamw_exact(oracle.bf16_widen(w16), m, v, gc, 3e-4, 0.9, 0.95, 1e-8, 0.1, 1)
    st = oracle.new_step_state()
    wo, mo, vo = w16.copy(), m.copy(), v.copy()
    oracle.adamw_bf16_step(wo, mo, vo, g16, st, lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1,
                           max_norm=1.0, spike_threshold=5.0, skip_steps=5)
    assert np.array_equal(wo, np.array([_bf16_round_exact(x) for x in wn], np.uint16))
    assert np.array_equal(_words(mo), _words(mn)) and np.array_equal(_words(vo), _words(vn))
