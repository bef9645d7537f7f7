"""GPU parity: repro_adamw_hash (the update and the state hash overlapped on
two streams) against the oracle and against the two calls in turn.

OPEN-1B paper, section 3.2 (the fused AdamW step) and Appendix B with
Figure 11 (the per-step BLAKE2b state hash, moved onto the device).
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


def _state(n, seed):
    w = synth.generate(n, synth.NORMAL, synth.tid(8, seed), 0.02)
    m = synth.generate(n, synth.NORMAL, synth.tid(8, seed + 1), 1e-4)
    v = synth.generate(n, synth.HALF_NORMAL, synth.tid(8, seed + 2), 1e-6)
    g = synth.generate(n, synth.NORMAL, synth.tid(8, seed + 3), 1e-3)
    return np.concatenate([w, m, v]), g


# chunk 0 with n a multiple of 1024: the single fused kernel (64 leaf
# triples per workgroup; 197 * 1024 leaves a partial last workgroup);
# chunk > 0: the two-stream pipeline; chunk < 0 or short n: in turn.
@pytest.mark.parametrize("n,chunk", [(5000, 0), (37 * 1024, 5 * 1024), (37 * 1024, 1024), (37 * 1024, -1),
                                     (64 * 1024, 16 * 1024), (3 * 1024, 0), (1024, 1024), (1024, 0),
                                     (37 * 1024, 0), (197 * 1024, 0), (128 * 1024, 0)])
def test_matches_oracle(n, chunk):
    st, g = _state(n, 16 + n % 7)
    ref = st.copy()
    oracle.adamw_inplace(ref, g, step=7, **HP)
    ref_digest = oracle.state_hash(ref)
    dst, dg = to_dev(st), to_dev(g)
    ws = br.hash_workspace(3 * n)
    digest = torch.empty(32, dtype=torch.uint8, device="cuda")
    br.repro_adamw_hash(dst, dg, digest, ws, step=7, chunk=chunk, **HP)
    assert_bitwise(to_host(dst), ref, f"state n={n} chunk={chunk}")
    assert bytes(digest.cpu().numpy().tobytes()) == ref_digest


def test_unaligned_view_takes_the_pipeline():
    n = 40 * 1024
    st, g = _state(n, 60)
    ref = st.copy()
    oracle.adamw_inplace(ref, g, step=2, **HP)
    big = to_dev(np.concatenate([[0], st]).astype(np.float32))
    dst = big[1:]  # 4-byte aligned only
    dg = to_dev(g)
    ws = br.hash_workspace(3 * n)
    digest = torch.empty(32, dtype=torch.uint8, device="cuda")
    br.repro_adamw_hash(dst, dg, digest, ws, step=2, **HP)
    assert_bitwise(to_host(dst), ref, "unaligned state")
    assert bytes(digest.cpu().numpy().tobytes()) == oracle.state_hash(ref)


@pytest.mark.parametrize("chunk", [0, 8 * 1024])
def test_steps_equal_the_two_calls_in_turn(chunk):
    n = 48 * 1024
    st, g = _state(n, 40)
    a, b = to_dev(st), to_dev(st)
    dg = to_dev(g)
    wa, wb = br.hash_workspace(3 * n), br.hash_workspace(3 * n)
    da = torch.empty(32, dtype=torch.uint8, device="cuda")
    db = torch.empty(32, dtype=torch.uint8, device="cuda")
    for step in range(1, 6):
        br.repro_adamw_hash(a, dg, da, wa, step=step, chunk=chunk, **HP)
        br.repro_adamw(b, dg, step=step, **HP)
        br.repro_state_hash_async(b, db, wb)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        assert torch.equal(da, db)


def test_other_stream_and_errors():
    n = 16 * 1024
    st, g = _state(n, 50)
    ref = st.copy()
    oracle.adamw_inplace(ref, g, step=3, **HP)
    s = torch.cuda.Stream()
    dst, dg = to_dev(st), to_dev(g)
    ws = br.hash_workspace(3 * n)
    digest = torch.empty(32, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        br.repro_adamw_hash(dst, dg, digest, ws, step=3, chunk=2048, stream=s, **HP)
    s.synchronize()
    assert_bitwise(to_host(dst), ref, "side stream")
    assert bytes(digest.cpu().numpy().tobytes()) == oracle.state_hash(ref)
    lib = br.library()
    p = dst.data_ptr()
    assert lib.repro_adamw_hash(p, dg.data_ptr(), n, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1, ws.data_ptr(), ws.numel(),
                                digest.data_ptr(), 1000, None) == -1  # chunk not a multiple of 1024
    assert lib.repro_adamw_hash(p, dg.data_ptr(), n, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1, ws.data_ptr(), 64,
                                digest.data_ptr(), 0, None) == -4
    assert lib.repro_adamw_hash(p, dg.data_ptr(), n, 1e-3, 0.9, 0.999, 1e-8, 0.1, 0, ws.data_ptr(), ws.numel(),
                                digest.data_ptr(), 0, None) == -1  # step < 1


def test_full_size_equals_the_two_calls():
    # The optimizer workload (n = 1.2e9, [w|m|v] 14.4 GB), fused kernel, and
    # the pipelined form on a third copy.
    AC = synth.ADAMW
    n = AC["n"]
    print(f"adamw+hash n={n}", flush=True)
    rng = np.random.default_rng(77)
    idx = np.unique(rng.integers(0, n, 4000))
    st = torch.empty(3 * n, dtype=torch.float32, device="cuda")
    parts = []
    for k, gen in enumerate((synth.adamw_w, synth.adamw_m, synth.adamw_v)):
        host = gen()
        parts.append(host[idx].copy())
        st[k * n:(k + 1) * n].copy_(torch.from_numpy(host))
        del host
    host = synth.adamw_g()
    g_sample = host[idx].copy()
    g = torch.from_numpy(host).cuda()
    del host
    other = st.clone()
    third = st.clone()
    ws = br.hash_workspace(3 * n)
    d1 = torch.empty(32, dtype=torch.uint8, device="cuda")
    d2 = torch.empty(32, dtype=torch.uint8, device="cuda")
    d3 = torch.empty(32, dtype=torch.uint8, device="cuda")
    hp = dict(lr=AC["lr"], beta1=AC["beta1"], beta2=AC["beta2"], eps=AC["eps"], weight_decay=AC["wd"])
    br.repro_adamw_hash(st, g, d1, ws, step=AC["step"], **hp)
    # Sampled leaves of the fused kernel's level 0 against the oracle, on the
    # updated words, and sampled elements of the update itself.
    nleaves = 3 * n // 1024
    leaves = sorted({0, n // 1024 - 1, n // 1024, 2 * n // 1024, nleaves - 1} |
                    set(rng.integers(0, nleaves, 11).tolist()))
    lvl0 = ws[:32 * nleaves].view(nleaves, 32)
    for leaf in leaves:
        words = st[leaf * 1024:(leaf + 1) * 1024].cpu().numpy()
        assert lvl0[leaf].cpu().numpy().tobytes() == oracle.state_hash_one_leaf(words, leaf, leaf == nleaves - 1), leaf
    sample = np.concatenate(parts).astype(np.float32)
    oracle.adamw_inplace(sample, g_sample, step=AC["step"], **hp)
    tidx = torch.from_numpy(idx).cuda()
    got = np.concatenate([st[:n][tidx].cpu().numpy(), st[n:2 * n][tidx].cpu().numpy(), st[2 * n:][tidx].cpu().numpy()])
    assert_bitwise(got, sample, "full-size fused update, sampled")
    br.repro_adamw(other, g, step=AC["step"], **hp)
    br.repro_state_hash_async(other, d2, ws)
    assert torch.equal(st.view(torch.int32), other.view(torch.int32))
    assert torch.equal(d1, d2)
    del other
    br.repro_adamw_hash(third, g, d3, ws, step=AC["step"], chunk=1 << 26, **hp)
    assert torch.equal(st.view(torch.int32), third.view(torch.int32))
    assert torch.equal(d1, d3)


def test_full_size_ten_repeats_and_the_oracle_digest():
    # The bench step's fused call on the optimizer workload, ten times from
    # the same state: ten identical digests, equal to the oracle's AdamW
    # followed by its single-threaded BLAKE2b over all 14.4 GB.
    AC = synth.ADAMW
    n = AC["n"]
    print(f"fused adamw+hash repeats n={n}", flush=True)
    host = np.empty(3 * n, np.float32)
    synth.adamw_w(n, out=host[:n])
    synth.adamw_m(n, out=host[n:2 * n])
    synth.adamw_v(n, out=host[2 * n:])
    g = synth.adamw_g()
    st0 = torch.from_numpy(host).cuda()
    dg = torch.from_numpy(g).cuda()
    ws = br.hash_workspace(3 * n)
    hp = dict(lr=AC["lr"], beta1=AC["beta1"], beta2=AC["beta2"], eps=AC["eps"], weight_decay=AC["wd"])
    digests = set()
    for _ in range(10):
        st = st0.clone()
        d = torch.empty(32, dtype=torch.uint8, device="cuda")
        br.repro_adamw_hash(st, dg, d, ws, step=AC["step"], **hp)
        digests.add(bytes(d.cpu().numpy().tobytes()))
        del st
    assert len(digests) == 1
    del st0
    oracle.adamw_inplace(host, g, step=AC["step"], **hp)
    print("oracle update done", flush=True)
    assert digests.pop() == oracle.state_hash(host)
