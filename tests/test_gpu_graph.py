"""The hot path under HIP graph capture: a captured step replays bit for bit.

Every entry point only enqueues kernels on the caller's stream (no device
allocation, no memset, no host synchronisation, no host-side state), so a
whole training step can be captured once and replayed.  The step here is
the tiny workload's chain (TreeFold of 4 replicas, a 64^3 GEMM, AdamW with
the state hash in one call) plus a BF16 optimizer step, whose step count,
skip window and beta powers live in device memory and so advance on every
replay.  Each replay is checked against the same calls made eagerly on
copies of the inputs, with eager work and a synchronisation in between
replays, and the last one against the oracle.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

BF16_HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, spike_threshold=5.0,
               skip_steps=5)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


class Step:
    """Buffers of one copy of the step and the step's calls on them."""

    def __init__(self, reps, dA, dB, state0, w16, m, v, g16, cfg):
        n = cfg["n"]
        self.reps, self.dA, self.dB = reps, dA, dB
        self.g_red = torch.empty(n, device="cuda")
        self.C = torch.empty(64, 64, device="cuda")
        self.state = to_dev(state0)
        self.digest = torch.zeros(32, dtype=torch.uint8, device="cuda")
        self.ws = br.hash_workspace(3 * n)
        self.w = torch.from_numpy(w16.view(np.int16)).cuda().view(torch.bfloat16)
        self.m, self.v = to_dev(m), to_dev(v)
        self.g16 = torch.from_numpy(g16.view(np.int16)).cuda().view(torch.bfloat16)
        self.bstate = br.new_step_state()
        self.bws = br.grad_norm_workspace(g16.size)
        self.hp = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"],
                       weight_decay=cfg["wd"])

    def run(self):
        br.repro_tree_reduce(self.reps, out=self.g_red)
        br.repro_gemm(self.dA, self.dB, out=self.C)
        br.repro_adamw_hash(self.state, self.g_red, self.digest, self.ws, step=7, **self.hp)
        br.repro_adamw_bf16_step(self.w, self.m, self.v, self.g16, self.bstate, workspace=self.bws, **BF16_HP)

    def host(self):
        return {"g_red": to_host(self.g_red), "C": to_host(self.C), "state": to_host(self.state),
                "digest": to_host(self.digest), "w": to_host(self.w.view(torch.int16)), "m": to_host(self.m),
                "v": to_host(self.v), "bstate": to_host(self.bstate)}


def test_captured_step_replays_bit_for_bit():
    cfg = synth.TINY
    n = cfg["n"]
    reps_h = [synth.tiny_replica(r) for r in range(cfg["R"])]
    reps = [to_dev(x) for x in reps_h]
    a, b = synth.tiny_gemm_inputs()
    dA, dB = to_dev(a), to_dev(b)
    state0 = np.concatenate([synth.tiny_adamw_weights(n), np.zeros(2 * n, np.float32)])
    nb = 100_003
    w16 = _bf16_bits(synth.generate(nb, synth.NORMAL, synth.tid(8, 0x10), 0.02))
    m = synth.generate(nb, synth.NORMAL, synth.tid(8, 0x11), 1e-4)
    v = np.abs(synth.generate(nb, synth.NORMAL, synth.tid(8, 0x12), 1e-6))
    g16 = _bf16_bits(synth.generate(nb, synth.NORMAL, synth.tid(8, 0x13), 1e-2))  # norm ~3.2: clipped
    args = (reps, dA, dB, state0, w16, m, v, g16, cfg)

    captured, eager, warm = Step(*args), Step(*args), Step(*args)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, on separate buffers
        warm.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured.run()
    torch.cuda.synchronize()
    for k in range(4):
        graph.replay()
        eager.run()
        torch.cuda.synchronize()
        got, ref = captured.host(), eager.host()
        for key in ref:
            assert np.array_equal(got[key].view(np.uint8), ref[key].view(np.uint8)), f"replay {k}: {key}"
        # Eager work of the program's own between replays.
        torch.cuda.synchronize()

    # The fourth replay against the oracle: four AdamW steps at t = 7 on the
    # fold, the hash of the result, and four BF16 steps.
    g_ref = oracle.tree_reduce(reps_h)
    assert_bitwise(got["g_red"], g_ref, "fold")
    assert_bitwise(got["C"], oracle.gemm(a, b), "gemm")
    st = state0
    for _ in range(4):
        st = oracle.adamw(st, g_ref, step=7, lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"],
                          weight_decay=cfg["wd"])
    assert_bitwise(got["state"], st, "state")
    assert bytes(got["digest"].tobytes()) == oracle.state_hash(st)
    wr, mr, vr = w16.copy(), m.copy(), v.copy()
    sr = oracle.new_step_state()
    for _ in range(4):
        oracle.adamw_bf16_step(wr, mr, vr, g16, sr, **BF16_HP)
    assert np.array_equal(got["w"].view(np.uint16), wr), "bf16 w"
    assert_bitwise(got["m"], mr, "bf16 m")
    assert_bitwise(got["v"], vr, "bf16 v")
    assert br.read_step_state(captured.bstate)["step"] == 4


def test_captured_no_allocation_update_and_hash():
    # The no-allocation AdamW + state hash is for callers that capture: its
    # digests live in the library's own array, so the captured graph holds
    # only kernels.  Three replays (each one more AdamW step at t = 7 on the
    # same state), each against the workspace form called eagerly on a copy.
    n = 1024 * 40
    st0 = np.concatenate([synth.generate(n, synth.NORMAL, synth.tid(8, 0x20), 0.02),
                          synth.generate(n, synth.NORMAL, synth.tid(8, 0x21), 1e-4),
                          np.abs(synth.generate(n, synth.NORMAL, synth.tid(8, 0x22), 1e-6))])
    g = synth.generate(n, synth.NORMAL, synth.tid(8, 0x23), 1e-3)
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=7)
    dg = to_dev(g)
    cap_state, eager_state, warm_state = to_dev(st0), to_dev(st0), to_dev(st0)
    cap_digest = torch.zeros(32, dtype=torch.uint8, device="cuda")
    eager_digest = torch.zeros(32, dtype=torch.uint8, device="cuda")
    ws = br.hash_workspace(3 * n)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first call (and the array's address lookup) outside the capture
        br.repro_adamw_hash_noalloc(warm_state, dg, torch.empty_like(cap_digest), **hp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        br.repro_adamw_hash_noalloc(cap_state, dg, cap_digest, **hp)
    torch.cuda.synchronize()
    ref = st0.copy()
    for k in range(3):
        graph.replay()
        br.repro_adamw_hash(eager_state, dg, eager_digest, ws, **hp)
        torch.cuda.synchronize()
        assert torch.equal(cap_state.view(torch.int32), eager_state.view(torch.int32)), f"replay {k}: state"
        assert torch.equal(cap_digest, eager_digest), f"replay {k}: digest"
        oracle.adamw_inplace(ref, g, **hp)
    assert_bitwise(to_host(cap_state), ref, "state after three replays")
    assert bytes(to_host(cap_digest).tobytes()) == oracle.state_hash(ref)


def test_captured_gemms_with_interior_tiles():
    # GEMMs whose interior tiles take the unchecked slab loads, captured and
    # replayed: 512 x 640 x 96 (128 x 128 tiles), 4096 x 4096 x 32 (512 tiles
    # of 256 x 128, the large-output kernel) and the fused convention on the
    # matrix cores, dW-style (trans_a).  Three replays, each against the same
    # calls made eagerly, then the oracle.
    shapes = [(512, 640, 96, 0, "unfused"), (4096, 4096, 32, 0, "unfused"), (512, 512, 64, 1, "fused")]
    ins = []
    for i, (M, N, K, ta, conv) in enumerate(shapes):
        A = synth.generate(M * K, synth.NORMAL, synth.tid(8, 0x30 + 2 * i), 1.0).reshape((K, M) if ta else (M, K))
        B = synth.generate(K * N, synth.NORMAL, synth.tid(8, 0x31 + 2 * i), 0.5).reshape(K, N)
        ins.append((A, B, to_dev(A), to_dev(B)))

    def run(outs):
        for (M, N, K, ta, conv), (_, _, dA, dB), C in zip(shapes, ins, outs):
            if conv == "fused":
                br.repro_gemm_fma(dA, dB, bool(ta), False, out=C, variant=0)
            else:
                br.repro_gemm(dA, dB, bool(ta), False, out=C)

    new = lambda: [torch.empty(M, N, device="cuda") for (M, N, _, _, _) in shapes]
    cap, eager, warm = new(), new(), new()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(warm)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(cap)
    torch.cuda.synchronize()
    for k in range(3):
        for C in cap:
            C.fill_(float("nan"))  # a replay must rewrite every word
        torch.cuda.synchronize()
        graph.replay()
        run(eager)
        torch.cuda.synchronize()
        for i, (C, E) in enumerate(zip(cap, eager)):
            assert torch.equal(C.view(torch.int32), E.view(torch.int32)), f"replay {k}: gemm {shapes[i]}"
    for (M, N, K, ta, conv), (A, B, _, _), C in zip(shapes, ins, cap):
        ref = oracle.gemm(A, B, bool(ta), False, fused=(conv == "fused"))
        assert_bitwise(to_host(C), ref, f"gemm {M}x{N}x{K} ta={ta} {conv}")
