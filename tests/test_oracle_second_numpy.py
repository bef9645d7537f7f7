"""A second, independent oracle for the tiny chained workload, written with
numpy float32 array arithmetic (CPU only).

Each numpy float32 operation is one IEEE binary32 operation rounded to
nearest-even, and numpy never fuses a multiply with an add, so this
re-derivation of the declared orders catches a C build of the oracle that
contracted or reordered anything.  numpy does not flush subnormals; the test
first checks that none arise anywhere in the workload, where the flush rule
has nothing to do.

OPEN-1B paper, section 2.1 (unfused MAC, one fixed order), Appendix A.1 and
A.3 (TreeFold, reciprocal average), section 3.2 (AdamW); RFC 7693 / hashlib
for the hash.
"""
import hashlib

import numpy as np

import oracle
import synth

F = np.float32
TINY = np.float32(2.0 ** -126)


def _no_subnormals(*arrays):
    for a in arrays:
        a = np.asarray(a, np.float32)
        assert not np.any((a != 0) & (np.abs(a) < TINY))


def gemm_np(A, B):
    M, K = A.shape
    acc = np.zeros((M, B.shape[1]), np.float32)
    for k in range(K):  # ascending k; each step one product and one sum
        p = A[:, k:k + 1] * B[k:k + 1, :]
        _no_subnormals(p, acc)
        acc = acc + p
    return acc


def treefold4_np(x):
    # R = 4: ((x0 + x1) + (x2 + x3)) * fl(1/4)
    s = (x[0] + x[1]) + (x[2] + x[3])
    return s * (F(1) / F(4))


def adamw_np(w, m, v, g, lr, b1, b2, eps, wd, step):
    b1, b2, lr, eps, wd = F(b1), F(b2), F(lr), F(eps), F(wd)
    c1, c2 = F(1) - b1, F(1) - b2
    p1, p2 = b1, b2
    for _ in range(step - 1):
        p1, p2 = p1 * b1, p2 * b2
    r1, r2 = F(1) / (F(1) - p1), F(1) / (F(1) - p2)
    m1 = b1 * m
    m2 = c1 * g
    mn = m1 + m2
    q = g * g
    v1 = b2 * v
    v2 = c2 * q
    vn = v1 + v2
    mh = mn * r1
    vh = vn * r2
    sq = np.sqrt(vh)
    d = sq + eps
    u = mh / d
    y = wd * w
    z = u + y
    t = lr * z
    wn = w - t
    _no_subnormals(m1, m2, mn, q, v1, v2, vn, mh, vh, sq, d, u, y, z, t, wn)
    return wn, mn, vn


def state_hash_hashlib(words):
    # BLAKE2b tree mode as declared: leaf 4096 B, fanout 16, depth 255, inner 32 B,
    # digest 32 B, personal "repro_state_v1"; last node flagged on every level.
    data = np.ascontiguousarray(words, np.float32).tobytes()
    leaves = [data[i:i + 4096] for i in range(0, len(data), 4096)] or [b""]
    level = [hashlib.blake2b(c, digest_size=32, fanout=16, depth=255, leaf_size=4096, node_offset=i,
                             node_depth=0, inner_size=32, last_node=(i == len(leaves) - 1),
                             person=b"repro_state_v1").digest() for i, c in enumerate(leaves)]
    depth = 1
    while True:
        groups = [b"".join(level[i:i + 16]) for i in range(0, len(level), 16)]
        level = [hashlib.blake2b(c, digest_size=32, fanout=16, depth=255, leaf_size=4096, node_offset=i,
                                 node_depth=depth, inner_size=32, last_node=(i == len(groups) - 1),
                                 person=b"repro_state_v1").digest() for i, c in enumerate(groups)]
        if len(level) == 1:
            return level[0]
        depth += 1


def test_tiny_chain_matches_the_c_oracle():
    cfg = synth.TINY
    a, b = synth.tiny_gemm_inputs()
    np.testing.assert_array_equal(gemm_np(a, b).view(np.uint32), oracle.gemm(a, b).view(np.uint32))
    reps = np.stack([synth.tiny_replica(r) for r in range(cfg["R"])])
    _no_subnormals(reps)
    g = treefold4_np(reps)
    np.testing.assert_array_equal(g.view(np.uint32), oracle.tree_reduce(list(reps)).view(np.uint32))
    n = cfg["n"]
    w = synth.tiny_adamw_weights(n)
    z = np.zeros(n, np.float32)
    wn, mn, vn = adamw_np(w, z, z, g, cfg["lr"], cfg["beta1"], cfg["beta2"], cfg["eps"], cfg["wd"], cfg["step"])
    st = oracle.adamw(np.concatenate([w, z, z]), g, cfg["lr"], cfg["beta1"], cfg["beta2"], cfg["eps"], cfg["wd"],
                      cfg["step"])
    np.testing.assert_array_equal(np.concatenate([wn, mn, vn]).view(np.uint32), st.view(np.uint32))
    assert state_hash_hashlib(st) == oracle.state_hash(st)


def test_a_later_adamw_step_matches_too():
    # Step 7 from nonzero moments (bias corrections with 6 serial multiplies).
    rng = np.random.default_rng(3)
    n = 4096
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32) + np.float32(1e-9)
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    wn, mn, vn = adamw_np(w, m, v, g, 3e-4, 0.9, 0.999, 1e-8, 0.1, 7)
    st = oracle.adamw(np.concatenate([w, m, v]), g, 3e-4, 0.9, 0.999, 1e-8, 0.1, 7)
    np.testing.assert_array_equal(np.concatenate([wn, mn, vn]).view(np.uint32), st.view(np.uint32))
