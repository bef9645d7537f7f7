#!/usr/bin/env python
"""Benchmark of the reproducible training-step operations on one MI355X.

One step is one pass of the whole hot path over the full synthetic workloads,
every input already resident in HBM:
  1. repro_tree_reduce   R = 8 replicas x 16,777,216 floats, x fl(1/8)
  2. repro_gemm          Y[8192x8192] = X[8192x2048] W[2048x8192]
  3. repro_adamw_hash    the AdamW update of the flat [w|m|v] (n = 1.2e9, step
                         counter advancing) and the BLAKE2b tree hash of the
                         updated 14.4 GB, in one kernel that hashes each block
                         as it is written
  4. repro_gemm          dW[2048x8192] = X^T dY, X[16384x2048], dY[16384x8192]
Each op is bracketed by HIP events on the stream it runs on.  `value` is the
GB/s of the memory-side work (reduce bytes, AdamW bytes and the hashed bytes
over the event time of ops 1 and 3; the hashed bytes are read from LDS, not
HBM, so `hbm_gbps` gives the rate of the bytes that cross HBM); the GEMMs
are reported in GFLOP/s beside it.  After the steps, and not part of them: repro_adamw and
repro_state_hash as separate calls ("ops_in_turn", each kernel's own
roofline), and under "next_rows" the audit replay of one step's reduction
(OPEN-1B section 6, Algorithm 1: 6 replicas x 8 shards x 6 microbatches over
an 8,388,608-float slice), the fused multiply-add GEMM convention
(repro_gemm_fma, matrix cores and VALU) and the BF16-parameter optimizer
step (norm, clip, update on n = 1.2e9).  Then the outputs are checked
against the CPU oracle (every word of the reduce output, sampled rows and
columns of the GEMMs, sampled AdamW elements replayed through every step,
sampled hash leaves, the replay and BF16 step on samples), and the oracle
itself is timed on a bounded sample as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--gemm-variants | --valu-rates]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bit-exact GB/s (reduce+AdamW+hash) and GFLOP/s (repro_gemm) vs roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
FP32_VECTOR_PEAK = 157.3       # TFLOP/s, vendor figure (FMA counted as 2 flops)
# VALU issue rate: 256 CUs x 128 fp32 lanes per clock x 2.4 GHz = 78.6 T
# lane-operations/s (the vendor fp32 figure is this rate times 2 flops per
# FMA), i.e. 0.5 wave-instructions per SIMD per clock.  The declared MAC is a
# multiply and an add, two lane-ops for two flops, so the GEMM's ceiling is
# 78.6 TFLOP/s.  The default GEMM forms the products on the matrix cores
# (one v_mfma_f32_32x32x1_2b_f32 per 2048 products, 64 busy cycles) and adds
# them on the VALU; the two units take turns (co-execution counter 0), so per
# SIMD 2048 MACs cost 64 + 64 cycles, the same 78.6 TFLOP/s ceiling.
# Full-rate opcodes (v_mul_f32, v_add_f32, v_xor_b32, v_lshrrev_b32, ...)
# reach it in either encoding; `bench.py --valu-rates` measures 0.47-0.48 for
# long streams of them.
VALU_LANE_OPS = 256 * 128 * 2.4e9
GEMM_PEAK_TFLOPS = VALU_LANE_OPS / 1e12
# BLAKE2b: per 128-byte block 12 rounds x 8 G.  The compiled compression
# (k_hash_leaves, gfx950) is 2001 VALU instructions: 802 v_xor_b32 and 46
# other full-rate ones, 577 v_lshl_add_u64 (one per 64-bit add) and 576
# v_alignbit_b32 (two per rotation by 24, 16 or 63); the rotation by 32 is a
# register swap.  The instruction audit in the tests checks these counts.
HASH_VALU_PER_BLOCK = 2001
HASH_VALU_HALF_RATE_PER_BLOCK = 1153   # v_lshl_add_u64 + v_alignbit_b32
# Bound 1 (the `peak` of the hash rows): one issue slot per VALU instruction
# at the VALU issue rate above.
HASH_INSTR_PER_BYTE = HASH_VALU_PER_BLOCK / 128
HASH_PEAK_GBS = VALU_LANE_OPS / HASH_INSTR_PER_BYTE / 1e9
# Bound 2 (reported beside it as `*_issue_model`), from `bench.py
# --valu-rates`: v_alignbit_b32 and v_lshl_add_u64 are half-rate opcodes
# (0.22-0.24 wave-instructions per SIMD per clock alone), and a stream that
# interleaves them with full-rate ones, as every G function does, issues all
# of its instructions at that half rate (0.23-0.24 for alternating
# v_alignbit_b32 / v_xor_b32; only a long full-rate run amortises a short
# cluster of half-rate ones).  So each hash instruction takes two slots.
HASH_SLOTS_PER_BYTE = 2 * HASH_INSTR_PER_BYTE
HASH_MODEL_PEAK_GBS = VALU_LANE_OPS / HASH_SLOTS_PER_BYTE / 1e9
# The AdamW update in the fused kernel: 190 VALU instructions per four
# elements (16 operations each, with the correctly rounded division and
# square-root sequences), 47.5 per element.  The issue model counts them at
# the half rate too: the fused kernel's waves interleave them with the hash.
ADAMW_INSTR_PER_ELEMENT = 47.5


def recorded_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, per
    op, kept only while the kernel source is the one the counters came from."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic_bench_step.md")
    out = {}
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return out
    for ln in lines:
        parts = ln.split()
        if len(parts) == 5 and parts[0] == "traffic":
            _, op, nbytes, src, sha = parts
            h = hashlib.sha256()
            try:
                for f in src.split("+"):  # the kernel's source and the headers it includes
                    h.update(open(os.path.join(ROOT, "bitwise_reproducible_amd", "csrc", f), "rb").read())
            except OSError:
                continue
            now = h.hexdigest()[:16]
            if now == sha:
                out[op] = int(nbytes)
    return out


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-verify", action="store_true", help="skip the oracle check after timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--gemm-variants", action="store_true",
                   help="only the forward and weight-gradient GEMM workloads, through repro_gemm variant 0 (the "
                        "default: matrix-core products, VALU adds), variant 4 (VALU multiply and add) and "
                        "repro_gemm_fma variant 0 (matrix cores), one warm-up and 5 timed calls each: the kernel "
                        "comparison, and the run the matrix-core co-execution counters are taken on")
    p.add_argument("--valu-rates", action="store_true",
                   help="only the VALU issue-rate streams of libvalu_rates.so (single-opcode streams and the "
                        "interleavings of full- and half-rate opcodes that the kernels contain) and the co-issue "
                        "of fp32 and bf16 matrix instructions with VALU adds: the measurements behind the ALU bounds")
    p.add_argument("--calibration-copy", action="store_true",
                   help="after timing, run one plain copy of 64 MiB (a one-replica fold without the average) whose "
                        "HBM counters calibrate the FETCH_SIZE / WRITE_SIZE readings of a profiling run")
    return p.parse_args()


class Upload:
    """Generate a synthetic tensor chunk by chunk into pinned host memory and
    copy each chunk to its device slice, optionally keeping sampled values."""

    def __init__(self, torch, chunk=1 << 26):
        self.torch = torch
        self.buf = torch.empty(chunk, dtype=torch.float32, pin_memory=True)
        self.chunk = chunk

    def fill(self, dst, gen, n, sample_idx=None):
        import numpy as np
        keep = None if sample_idx is None else np.empty(sample_idx.size, np.float32)
        host = self.buf.numpy()
        for off in range(0, n, self.chunk):
            m = min(self.chunk, n - off)
            gen(m, offset=off, out=host[:m])
            dst[off:off + m].copy_(self.buf[:m], non_blocking=False)
            if keep is not None:
                lo, hi = np.searchsorted(sample_idx, [off, off + m])
                keep[lo:hi] = host[sample_idx[lo:hi] - off]
        return keep


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; the library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Reduce, AdamW and the hash would shard by contiguous element ranges and the GEMM by output "
              "tiles, with no change of bits.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import bitwise_reproducible_amd as br
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.gemm_variants:
        gemm_variants(torch, np, br, synth, dev)
        return
    if args.valu_rates:
        valu_rates()
        return
    up = Upload(torch)
    t_setup = time.time()

    # 1. Gradient reduction workload.
    RC = synth.REDUCE
    reps = []
    for r in range(RC["R"]):
        d = torch.empty(RC["n"], dtype=torch.float32, device=dev)
        up.fill(d, lambda m, offset, out, r=r: synth.reduce_replica(r, m, offset=offset, out=out), RC["n"])
        reps.append(d)
    g_red = torch.empty(RC["n"], dtype=torch.float32, device=dev)
    # 2. Forward GEMM workload.
    GC = synth.GEMM
    X3 = torch.empty(GC["M"] * GC["K"], dtype=torch.float32, device=dev)
    W3 = torch.empty(GC["K"] * GC["N"], dtype=torch.float32, device=dev)
    up.fill(X3, lambda m, offset, out: synth.generate(m, synth.NORMAL, synth.tid(3, 0), 1.0, offset=offset, out=out),
            X3.numel())
    up.fill(W3, lambda m, offset, out: synth.generate(m, synth.NORMAL, synth.tid(3, 1), 0.02, offset=offset,
                                                      out=out), W3.numel())
    X3 = X3.view(GC["M"], GC["K"])
    W3 = W3.view(GC["K"], GC["N"])
    Y3 = torch.empty(GC["M"], GC["N"], dtype=torch.float32, device=dev)
    # 3-4. Optimizer + hash workload.
    AC = synth.ADAMW
    n = AC["n"]
    rng = np.random.default_rng(12)
    aidx = np.unique(np.concatenate([np.arange(0, 1024), np.arange(n - 1024, n), rng.integers(0, n, 60_000)]))
    state = torch.empty(3 * n, dtype=torch.float32, device=dev)
    grad = torch.empty(n, dtype=torch.float32, device=dev)
    log(f"generating the optimizer state, 3 x {n} + {n} floats")
    s_w = up.fill(state[:n], lambda m, offset, out: synth.adamw_w(m, offset=offset, out=out), n, aidx)
    s_m = up.fill(state[n:2 * n], lambda m, offset, out: synth.adamw_m(m, offset=offset, out=out), n, aidx)
    s_v = up.fill(state[2 * n:], lambda m, offset, out: synth.adamw_v(m, offset=offset, out=out), n, aidx)
    s_g = up.fill(grad, lambda m, offset, out: synth.adamw_g(m, offset=offset, out=out), n, aidx)
    ws = br.hash_workspace(3 * n, dev)
    digest = torch.empty(32, dtype=torch.uint8, device=dev)
    # 5. Weight-gradient workload.
    DC = synth.DW
    X5 = torch.empty(DC["K"] * DC["M"], dtype=torch.float32, device=dev)
    dY5 = torch.empty(DC["K"] * DC["N"], dtype=torch.float32, device=dev)
    up.fill(X5, lambda m, offset, out: synth.generate(m, synth.STUDENT_T3, synth.tid(5, 0), 1e-2, offset=offset,
                                                      out=out), X5.numel())
    up.fill(dY5, lambda m, offset, out: synth.generate(m, synth.STUDENT_T3, synth.tid(5, 1), 1e-2, offset=offset,
                                                       out=out), dY5.numel())
    X5 = X5.view(DC["K"], DC["M"])
    dY5 = dY5.view(DC["K"], DC["N"])
    dW5 = torch.empty(DC["M"], DC["N"], dtype=torch.float32, device=dev)
    # Audit replay workload (timed after the steps).
    PC = synth.REPLAY
    p_layout = (PC["dp_replicate"], PC["dp_shard"], PC["accum"])
    p_nbuf = p_layout[0] * p_layout[1] * p_layout[2]
    p_grads = []
    for b in range(p_nbuf):
        d = torch.empty(PC["n"], dtype=torch.float32, device=dev)
        up.fill(d, lambda m, offset, out, b=b: synth.replay_grad(b, m, offset=offset, out=out), PC["n"])
        p_grads.append(d)
    p_out = torch.empty(PC["n"], dtype=torch.float32, device=dev)
    # BF16-parameter optimizer step workload (timed after the steps): the
    # same n, w bf16, FP32 moments, a bf16 gradient of norm ~3.5 (clipped).
    bidx = aidx
    b_w = torch.empty(n, dtype=torch.bfloat16, device=dev)
    b_g = torch.empty(n, dtype=torch.bfloat16, device=dev)
    b_m = torch.empty(n, dtype=torch.float32, device=dev)
    b_v = torch.empty(n, dtype=torch.float32, device=dev)
    tmp = torch.empty(up.chunk, dtype=torch.float32, device=dev)
    b_samples = {}
    for name, dst, gen in (("w", b_w, lambda m_, offset, out: synth.adamw_w(m_, offset=offset, out=out)),
                           ("g", b_g, lambda m_, offset, out: synth.generate(m_, synth.NORMAL, synth.tid(7, 3), 1e-4,
                                                                             offset=offset, out=out))):
        for off in range(0, n, up.chunk):
            m_ = min(up.chunk, n - off)
            up.fill(tmp[:m_], lambda mm, offset, out, off=off, gen=gen: gen(mm, offset=off + offset, out=out), m_)
            dst[off:off + m_].copy_(tmp[:m_])  # round to bf16 (input preparation)
        b_samples[name] = dst[torch.from_numpy(bidx).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    b_samples["m"] = up.fill(b_m, lambda m_, offset, out: synth.adamw_m(m_, offset=offset, out=out), n, bidx)
    b_samples["v"] = up.fill(b_v, lambda m_, offset, out: synth.adamw_v(m_, offset=offset, out=out), n, bidx)
    del tmp
    b_state = br.new_step_state(dev)
    b_ws = br.grad_norm_workspace(n, dev)
    torch.cuda.synchronize()
    del up
    log(f"inputs resident in HBM after {time.time() - t_setup:.1f} s")

    hp = dict(lr=AC["lr"], beta1=AC["beta1"], beta2=AC["beta2"], eps=AC["eps"], weight_decay=AC["wd"])
    ops = ["tree_reduce", "gemm_fwd", "adamw_state_hash", "gemm_dw"]
    step_counter = [AC["step"]]

    def one_step(events=None):
        rec = (lambda i: events[i].record()) if events else (lambda i: None)
        rec(0)
        br.repro_tree_reduce(reps, out=g_red)
        rec(1)
        br.repro_gemm(X3, W3, out=Y3)
        rec(2)
        br.repro_adamw_hash(state, grad, digest, ws, step=step_counter[0], **hp)  # update + hash, one kernel
        step_counter[0] += 1
        rec(3)
        br.repro_gemm(X5, dY5, trans_a=True, out=dW5)
        rec(4)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        one_step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    op_samples = {op: [evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)] for i, op in enumerate(ops)}
    op_ms = {op: float(np.mean(v)) for op, v in op_samples.items()}
    # Digests of every op's output after the last step (untimed; state hash
    # of the words).  With the same --steps and --warmup they are the same on
    # every run, box and process.
    dg_ws = br.hash_workspace(RC["n"] if RC["n"] > GC["M"] * GC["N"] else GC["M"] * GC["N"], dev)
    digests = {"steps_taken": args.warmup + args.steps,
               "tree_reduce_out": br.repro_state_hash(g_red, dg_ws).hex(),
               "gemm_fwd_out": br.repro_state_hash(Y3.view(-1), dg_ws).hex(),
               "gemm_dw_out": br.repro_state_hash(dW5.view(-1), dg_ws).hex(),
               "adamw_state": bytes(digest.cpu().numpy().tobytes()).hex()}
    del dg_ws

    # The replay, timed on its own: same warmup and count as the steps.
    for _ in range(args.warmup):
        br.repro_replay_reduce(p_grads, *p_layout, out=p_out)
    p_evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    p_evs[0].record()
    for s in range(args.steps):
        br.repro_replay_reduce(p_grads, *p_layout, out=p_out)
        p_evs[s + 1].record()
    torch.cuda.synchronize()
    replay_ms = float(np.mean([p_evs[s].elapsed_time(p_evs[s + 1]) for s in range(args.steps)]))

    # The fused multiply-add GEMM convention (declared alternative), both
    # workloads, matrix cores (variant 0) and VALU (variant 1).
    Y3f = torch.empty_like(Y3)
    dW5f = torch.empty_like(dW5)
    fma_ms = {}
    for variant in (0, 1):
        for name, call in (("fwd", lambda v: br.repro_gemm_fma(X3, W3, out=Y3f, variant=v)),
                           ("dw", lambda v: br.repro_gemm_fma(X5, dY5, trans_a=True, out=dW5f, variant=v))):
            for _ in range(args.warmup):
                call(variant)
            f_evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            torch.cuda.synchronize()
            f_evs[0].record()
            for s_ in range(args.steps):
                call(variant)
                f_evs[s_ + 1].record()
            torch.cuda.synchronize()
            fma_ms[(variant, name)] = float(np.mean([f_evs[i].elapsed_time(f_evs[i + 1])
                                                     for i in range(args.steps)]))

    # AdamW, then the state hash, as separate calls (repro_adamw,
    # repro_state_hash), for each kernel's own roofline: on a copy of the
    # optimizer state that continues from the steps' last step counter.
    state2 = state.clone()
    ws2 = br.hash_workspace(3 * n, dev)  # the steps' leaf digests in ws are checked later
    digest2 = torch.empty(32, dtype=torch.uint8, device=dev)
    ah_step0 = step_counter[0]
    for _ in range(args.warmup):
        br.repro_adamw(state2, grad, step=step_counter[0], **hp)
        br.repro_state_hash_async(state2, digest2, ws2)
        step_counter[0] += 1
    ah_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        ah_evs[s_][0].record()
        br.repro_adamw(state2, grad, step=step_counter[0], **hp)
        step_counter[0] += 1
        ah_evs[s_][1].record()
        br.repro_state_hash_async(state2, digest2, ws2)
        ah_evs[s_][2].record()
    torch.cuda.synchronize()
    turn_ms = {"adamw": float(np.mean([e[0].elapsed_time(e[1]) for e in ah_evs])),
               "state_hash": float(np.mean([e[1].elapsed_time(e[2]) for e in ah_evs]))}

    # The BF16 optimizer step, timed on its own.
    bhp = dict(lr=AC["lr"], beta1=0.9, beta2=0.95, eps=AC["eps"], weight_decay=AC["wd"], max_norm=1.0,
               spike_threshold=5.0, skip_steps=5)
    for _ in range(args.warmup):
        br.repro_adamw_bf16_step(b_w, b_m, b_v, b_g, b_state, workspace=b_ws, **bhp)
    b_evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    b_evs[0].record()
    for s_ in range(args.steps):
        br.repro_adamw_bf16_step(b_w, b_m, b_v, b_g, b_state, workspace=b_ws, **bhp)
        b_evs[s_ + 1].record()
    torch.cuda.synchronize()
    bf16_ms = float(np.mean([b_evs[i].elapsed_time(b_evs[i + 1]) for i in range(args.steps)]))

    if args.calibration_copy:
        br.repro_tree_reduce([reps[0]], out=g_red, average=False)
        torch.cuda.synchronize()

    # A plain copy for the secondary fractions: the one-replica fold without
    # the average reads and writes each word once (2 GiB in, 2 GiB out).
    copy_n = 1 << 29
    c_src = torch.ones(copy_n, dtype=torch.float32, device=dev)
    c_dst = torch.empty_like(c_src)
    c_ms = []
    for i in range(3 + 10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        br.repro_tree_reduce([c_src], out=c_dst, average=False)
        e1.record()
        c_ms.append((e0, e1))
    torch.cuda.synchronize()
    copy_ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in c_ms[3:]]))
    copy_gbps = 8 * copy_n / (copy_ms * 1e-3) / 1e9
    del c_src, c_dst

    # Algorithmic work per launch.
    bytes_reduce = (RC["R"] + 1) * 4 * RC["n"]
    bytes_adamw = 28 * n
    bytes_hash = 12 * n
    flops_fwd = 2 * GC["M"] * GC["N"] * GC["K"]
    flops_dw = 2 * DC["M"] * DC["N"] * DC["K"]
    mem_ms = op_ms["tree_reduce"] + op_ms["adamw_state_hash"]
    value = (bytes_reduce + bytes_adamw + bytes_hash) / (mem_ms * 1e-3) / 1e9
    # The bytes of those two ops that cross HBM: the reduce's, the update's
    # 28n and the leaf and inner digests written (the fused kernel hashes the
    # updated state from LDS, so the 12n hashed bytes are not read again).
    bytes_digests = br.repro_state_hash_workspace_bytes(3 * n)
    hbm_gbps = (bytes_reduce + bytes_adamw + bytes_digests) / (mem_ms * 1e-3) / 1e9
    gemm_ms = op_ms["gemm_fwd"] + op_ms["gemm_dw"]
    gemm_gflops = (flops_fwd + flops_dw) / (gemm_ms * 1e-3) / 1e9

    def roof(op, ms):
        if op in ("gemm_fwd", "gemm_dw"):
            f = flops_fwd if op == "gemm_fwd" else flops_dw
            ach = f / (ms * 1e-3) / 1e12
            return {"bound": "alu", "achieved": round(ach, 3), "peak": round(GEMM_PEAK_TFLOPS, 2),
                    "unit": "TFLOP/s", "frac": round(ach / GEMM_PEAK_TFLOPS, 4), "traffic": None,
                    "frac_of_fp32_vector_peak": round(ach / FP32_VECTOR_PEAK, 4)}
        if op == "adamw_state_hash":
            # One kernel, bound by the tighter of HBM (28n bytes) and the VALU
            # issue of the hash plus the update (instructions per element).
            t_hbm = bytes_adamw / (HBM_PEAK_GBS * 1e9)
            t_alu = n * (12 * HASH_INSTR_PER_BYTE + ADAMW_INSTR_PER_ELEMENT) / VALU_LANE_OPS
            t_model = n * (12 * HASH_SLOTS_PER_BYTE + 2 * ADAMW_INSTR_PER_ELEMENT) / VALU_LANE_OPS
            t_bound = max(t_hbm, t_alu)
            peak = bytes_hash / t_bound / 1e9
            ach = bytes_hash / (ms * 1e-3) / 1e9
            return {"bound": "alu" if t_alu >= t_hbm else "hbm", "achieved": round(ach, 1), "peak": round(peak, 1),
                    "unit": "GB/s (of state hashed)", "frac": round(t_bound / (ms * 1e-3), 4), "traffic": None,
                    "bound_ms": {"hbm": round(t_hbm * 1e3, 3), "alu_one_slot": round(t_alu * 1e3, 3),
                                 "alu_issue_model": round(t_model * 1e3, 3)},
                    "frac_issue_model": round(max(t_hbm, t_model) / (ms * 1e-3), 4),
                    "hbm_achieved": round(bytes_adamw / (ms * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(bytes_adamw / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "hbm_frac_of_copy": round(bytes_adamw / (ms * 1e-3) / 1e9 / copy_gbps, 4)}
        b = {"tree_reduce": bytes_reduce, "adamw": bytes_adamw, "state_hash": bytes_hash}[op]
        ach = b / (ms * 1e-3) / 1e9
        if op == "state_hash":  # integer-VALU bound: 15.6 instructions per byte
            return {"bound": "alu", "achieved": round(ach, 1), "peak": round(HASH_PEAK_GBS, 1), "unit": "GB/s",
                    "frac": round(ach / HASH_PEAK_GBS, 4), "traffic": None,
                    "peak_issue_model": round(HASH_MODEL_PEAK_GBS, 1),
                    "frac_issue_model": round(ach / HASH_MODEL_PEAK_GBS, 4),
                    "frac_of_hbm_peak": round(ach / HBM_PEAK_GBS, 4)}
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "frac_of_copy": round(ach / copy_gbps, 4)}

    per_op = {op: {"ms": round(op_ms[op], 4), "ms_median": round(float(np.median(op_samples[op])), 4),
                   "ms_min": round(float(np.min(op_samples[op])), 4), **roof(op, op_ms[op])} for op in ops}
    in_turn = {op: {"ms": round(turn_ms[op], 4), **roof(op, turn_ms[op])} for op in ("adamw", "state_hash")}
    traffic = recorded_traffic()
    for op in ops:
        per_op[op]["traffic"] = traffic.get(op)
    for op in in_turn:
        in_turn[op]["traffic"] = traffic.get("state_hash_leaves" if op == "state_hash" else op)
    dominant = max(ops, key=lambda o: op_ms[o])
    bytes_replay = (p_nbuf + 1) * 4 * PC["n"]
    ach = bytes_replay / (replay_ms * 1e-3) / 1e9
    next_rows = {"replay_reduce": {
        "workload": f"dp_replicate={p_layout[0]} dp_shard={p_layout[1]} accum={p_layout[2]} "
                    f"({p_nbuf} buffers) n={PC['n']}",
        "ms": round(replay_ms, 4), "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic.get("replay_reduce"),
        "frac_of_copy": round(ach / copy_gbps, 4)}}
    bytes_bf16 = 24 * n  # norm pass reads g (2n); update reads w, m, v, g (12n), writes w, m, v (10n)
    ach = bytes_bf16 / (bf16_ms * 1e-3) / 1e9
    next_rows["adamw_bf16_step"] = {
        "workload": f"n={n} bf16 w, fp32 m and v, bf16 g (norm ~3.5, clipped to 1.0), beta2 0.95",
        "ms": round(bf16_ms, 4), "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic.get("adamw_bf16_step"),
        "frac_of_copy": round(ach / copy_gbps, 4)}
    for variant, unit in ((0, "matrix cores, v_mfma_f32_32x32x1_2b_f32"), (1, "VALU, v_fma_f32")):
        ms = fma_ms[(variant, "fwd")] + fma_ms[(variant, "dw")]
        ach = (flops_fwd + flops_dw) / (ms * 1e-3) / 1e12
        next_rows[f"gemm_fma_variant{variant}"] = {
            "workload": "fused-MAC chains: gemm 8192x2048 @ 2048x8192 and dW 2048x8192 K=16384", "unit": unit,
            "ms_fwd": round(fma_ms[(variant, "fwd")], 4), "ms_dw": round(fma_ms[(variant, "dw")], 4),
            "bound": "mfma" if variant == 0 else "alu", "achieved": round(ach, 3), "peak": FP32_VECTOR_PEAK,
            "unit_rate": "TFLOP/s", "frac": round(ach / FP32_VECTOR_PEAK, 4)}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded Philox4x64-10, one counter-based stream per tensor)",
        "config": {"workload": "reduce R=8 n=16777216; gemm 8192x2048 @ 2048x8192; adamw+state_hash n=1.2e9 "
                               "[w|m|v] 14.4 GB; dW 2048x8192 K=16384",
                   "parallelism": "none (1 GPU)"},
        "value_counts": "algorithmic bytes of reduce + AdamW + hash: (R+1)*4n_reduce + 28n + 12n hashed, over the "
                        "event time of the reduce and the fused AdamW + hash; the 12n hashed bytes are read from LDS, "
                        "not HBM (see hbm_gbps)",
        "hbm_gbps": round(hbm_gbps, 1),
        "hbm_frac": round(hbm_gbps / HBM_PEAK_GBS, 4),
        "gemm": {"value": round(gemm_gflops, 1), "unit": "GFLOP/s"},
        "hbm_copy": {"gbps": round(copy_gbps, 1), "ms_median": round(copy_ms, 4), "bytes": 8 * copy_n,
                     "kernel": "k_tree_reduce_v4<1, false> (one-replica fold: a plain copy)"},
        "ops": per_op,
        "ops_in_turn": in_turn,
        "roofline": {"kernel": dominant, **{k: v for k, v in per_op[dominant].items() if not k.startswith("ms")}},
        "next_rows": next_rows,
        "digests": digests,
    }

    if not args.no_verify:
        out["verified"] = verify(torch, np, br, reps, g_red, X3, W3, Y3, X5, dY5, dW5, state, ws, n, aidx,
                                 (s_w, s_m, s_v, s_g), hp, AC["step"], args.warmup + args.steps)
        out["verified"].update(verify_replay(np, p_out, p_layout, PC["n"]))
        out["verified"].update(verify_fused(np, X3, W3, Y3f, X5, dY5, dW5f))
        out["verified"].update(verify_in_turn(np, torch, br, state2, digest2, ws2, n, aidx, (s_w, s_m, s_v, s_g),
                                              hp, AC["step"], step_counter[0]))
        out["verified"].update(verify_bf16(np, torch, br, b_g, b_w, b_m, b_v, b_state, bidx, b_samples, bhp,
                                           args.warmup + args.steps))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(np)
    print(json.dumps(out), flush=True)


def valu_rates():
    """Wave-instructions per SIMD per shader clock of the streams in
    libvalu_rates.so, with 2 and 4 waves on every SIMD."""
    import ctypes
    path = os.path.join(ROOT, "bitwise_reproducible_amd", "libvalu_rates.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    lib.valu_rates_name.restype = ctypes.c_char_p
    lib.valu_rates_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    out = []
    for s in range(lib.valu_rates_count()):
        name = lib.valu_rates_name(s).decode()
        row = {"stream": name}
        for w in (2, 4):
            res = (ctypes.c_double * 3)()
            rc = lib.valu_rates_run(s, w, 20000, res)
            if rc != 0:
                raise RuntimeError(f"valu_rates_run({name}, {w}) returned {rc}")
            row[f"w{w}"] = {"rate": round(res[0], 4), "ghz": round(res[1], 3), "ms": round(res[2], 3)}
        log(row)
        out.append(row)
    # Matrix-core / VALU co-issue: one wave of each role on every SIMD, the
    # passes sized so that each role alone runs about 1 ms.  overlap is
    # (matrix alone + VALU alone - both) / min(alone): 1 when the two issue
    # side by side, 0 when they take turns.
    lib.valu_rates_coissue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    co = []
    for kind, name, iters_m in ((0, "v_mfma_f32_32x32x1_2b_f32 (fp32)", 8000), (1, "v_mfma_f32_32x32x8_bf16", 16000)):
        res = (ctypes.c_double * 3)()
        rc = lib.valu_rates_coissue(kind, iters_m, 4000, res)
        if rc != 0:
            raise RuntimeError(f"valu_rates_coissue({kind}) returned {rc}")
        both, m, v = res[0], res[1], res[2]
        row = {"matrix": name, "with": "v_add_f32_e32", "ms_both": round(both, 3), "ms_matrix_alone": round(m, 3),
               "ms_valu_alone": round(v, 3), "overlap": round((m + v - both) / min(m, v), 3)}
        log(row)
        co.append(row)
    print(json.dumps({"valu_rates": out, "unit": "wave-instructions per SIMD per shader clock", "coissue": co}),
          flush=True)


def gemm_variants(torch, np, br, synth, dev, reps=5):
    """The forward and weight-gradient GEMM workloads through the default
    kernel (matrix-core products, VALU adds), the VALU multiply-and-add
    kernel, and the fused matrix-core kernel: one warm-up call, then `reps`
    calls timed one by one with events (median and min).  The unfused
    variants must give the same digest."""
    up = Upload(torch)
    GC, DC = synth.GEMM, synth.DW
    X3 = torch.empty(GC["M"] * GC["K"], dtype=torch.float32, device=dev)
    W3 = torch.empty(GC["K"] * GC["N"], dtype=torch.float32, device=dev)
    up.fill(X3, lambda m, offset, out: synth.generate(m, synth.NORMAL, synth.tid(3, 0), 1.0, offset=offset, out=out),
            X3.numel())
    up.fill(W3, lambda m, offset, out: synth.generate(m, synth.NORMAL, synth.tid(3, 1), 0.02, offset=offset,
                                                      out=out), W3.numel())
    X5 = torch.empty(DC["K"] * DC["M"], dtype=torch.float32, device=dev)
    dY5 = torch.empty(DC["K"] * DC["N"], dtype=torch.float32, device=dev)
    up.fill(X5, lambda m, offset, out: synth.generate(m, synth.STUDENT_T3, synth.tid(5, 0), 1e-2, offset=offset,
                                                      out=out), X5.numel())
    up.fill(dY5, lambda m, offset, out: synth.generate(m, synth.STUDENT_T3, synth.tid(5, 1), 1e-2, offset=offset,
                                                       out=out), dY5.numel())
    X3, W3 = X3.view(GC["M"], GC["K"]), W3.view(GC["K"], GC["N"])
    X5, dY5 = X5.view(DC["K"], DC["M"]), dY5.view(DC["K"], DC["N"])
    Y = torch.empty(max(GC["M"] * GC["N"], DC["M"] * DC["N"]), dtype=torch.float32, device=dev)
    Y3, Y5 = Y[:GC["M"] * GC["N"]].view(GC["M"], GC["N"]), Y[:DC["M"] * DC["N"]].view(DC["M"], DC["N"])
    shapes = {"fwd": (lambda f, v: f(X3, W3, out=Y3, variant=v), Y3, 2.0 * GC["M"] * GC["N"] * GC["K"]),
              "dw": (lambda f, v: f(X5, dY5, trans_a=True, out=Y5, variant=v), Y5, 2.0 * DC["M"] * DC["N"] * DC["K"])}
    kernels = {"repro_gemm_variant0": (br.repro_gemm, 0), "repro_gemm_variant4": (br.repro_gemm, 4),
               "repro_gemm_fma_variant0": (br.repro_gemm_fma, 0)}
    out = {}
    for shape, (call, Yv, flops) in shapes.items():
        for name, (f, v) in kernels.items():
            call(f, v)
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call(f, v)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            med = float(np.median(ts))
            out[f"{shape}_{name}"] = {"ms_median": round(med, 4), "ms_min": round(min(ts), 4),
                                      "tflops": round(flops / med / 1e9, 2),
                                      "digest": br.repro_state_hash(Yv.reshape(-1)).hex()}
            log(shape, name, out[f"{shape}_{name}"])
        if out[f"{shape}_repro_gemm_variant0"]["digest"] != out[f"{shape}_repro_gemm_variant4"]["digest"]:
            raise RuntimeError(f"{shape}: the unfused variants gave different bits")
    print(json.dumps({"gemm_variants": out, "workloads": {"fwd": "8192x2048 @ 2048x8192",
                                                          "dw": "(16384x2048)^T @ 16384x8192"}}), flush=True)


def verify(torch, np, br, reps, g_red, X3, W3, Y3, X5, dY5, dW5, state, ws, n, aidx, samples, hp, step0, nsteps):
    """Bit-exactness of the timed run's outputs against the oracle (sampled)."""
    import oracle

    def differing_words(a, b):
        a = np.ascontiguousarray(a, np.float32).reshape(-1).view(np.uint32)
        b = np.ascontiguousarray(b, np.float32).reshape(-1).view(np.uint32)
        return np.nonzero(a != b)[0]

    t = time.time()
    res = {}
    reps_h = [r.cpu().numpy() for r in reps]
    res["tree_reduce_words_differing"] = int(differing_words(g_red.cpu().numpy(), oracle.tree_reduce(reps_h)).size)
    del reps_h

    def gemm_rows_cols(A_op, Bt, C, rows, cols):
        bad = 0
        for r in rows:
            bad += differing_words(C[r].cpu().numpy(), oracle.gemm(A_op[r:r + 1], Bt, trans_b=True)[0]).size
        for c in cols:
            bad += differing_words(C[:, c].cpu().numpy(), oracle.gemm(A_op, Bt[c:c + 1], trans_b=True)[:, 0]).size
        return int(bad)

    a3 = X3.cpu().numpy()
    bt3 = np.ascontiguousarray(W3.cpu().numpy().T)
    res["gemm_fwd_sampled_words_differing"] = gemm_rows_cols(a3, bt3, Y3, [0, 4097], [8191])
    a5 = np.ascontiguousarray(X5.cpu().numpy().T)
    bt5 = np.ascontiguousarray(dY5.cpu().numpy().T)
    res["gemm_dw_sampled_words_differing"] = gemm_rows_cols(a5, bt5, dW5, [1029], [77])
    del a3, bt3, a5, bt5
    # AdamW: replay every step the GPU took on the sampled elements.
    s_w, s_m, s_v, s_g = samples
    st = np.concatenate([s_w, s_m, s_v]).astype(np.float32)
    for t_ in range(step0, step0 + nsteps):
        oracle.adamw_inplace(st, s_g, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], t_)
    tidx = torch.from_numpy(aidx).to(state.device)
    k = aidx.size
    got = np.concatenate([state[:n][tidx].cpu().numpy(), state[n:2 * n][tidx].cpu().numpy(),
                          state[2 * n:][tidx].cpu().numpy()])
    res["adamw_sampled_words_differing"] = int(differing_words(got, st).size)
    res["adamw_sampled_elements"] = int(k)
    # Hash: leaf digests of the final state at sampled leaves (level 0 of the workspace).
    nleaves = (12 * n + 4095) // 4096
    leaves = sorted({0, 1, nleaves // 3, nleaves // 3 + 1, nleaves - 1} |
                    set(np.random.default_rng(5).integers(0, nleaves, 27).tolist()))
    wsh = ws[:32 * nleaves].view(nleaves, 32)
    bad = 0
    for leaf in leaves:
        words = state[leaf * 1024:(leaf + 1) * 1024].cpu().numpy()
        ref = oracle.state_hash_one_leaf(words, leaf, leaf == nleaves - 1)
        bad += int(wsh[leaf].cpu().numpy().tobytes() != ref)
    res["state_hash_sampled_leaves_differing"] = bad
    res["state_hash_sampled_leaves"] = len(leaves)
    res["seconds"] = round(time.time() - t, 1)
    return res


def verify_replay(np, p_out, layout, n):
    """The replay output against the oracle on three regenerated slices."""
    import oracle
    import synth
    t = time.time()
    nbuf = layout[0] * layout[1] * layout[2]
    m = 1 << 16
    starts = [0, int(np.random.default_rng(9).integers(1, n // m - 1)) * m + 12_345, n - m]
    bad = 0
    for s0 in starts:
        grads = [synth.replay_grad(b, m, offset=s0) for b in range(nbuf)]
        ref = oracle.replay_reduce(grads, *layout)
        got = p_out[s0:s0 + m].cpu().numpy()
        bad += int(np.count_nonzero(got.view(np.uint32) != ref.view(np.uint32)))
    return {"replay_sampled_words_differing": bad, "replay_sampled_words": len(starts) * m,
            "replay_seconds": round(time.time() - t, 1)}


def verify_fused(np, X3, W3, Y3f, X5, dY5, dW5f):
    """The last fused GEMM outputs (VALU variant) against the oracle's fused
    chains on sampled rows and columns."""
    import oracle
    t = time.time()
    bad = 0
    x3 = X3.cpu().numpy()
    bt3 = np.ascontiguousarray(W3.cpu().numpy().T)
    y = Y3f.cpu().numpy()
    bad += int(np.count_nonzero(y[4097].view(np.uint32) !=
                                oracle.gemm(x3[4097:4098], bt3, trans_b=True, fused=True)[0].view(np.uint32)))
    bad += int(np.count_nonzero(y[:, 8191].view(np.uint32) !=
                                oracle.gemm(x3, bt3[8191:], trans_b=True, fused=True)[:, 0].view(np.uint32)))
    a5 = np.ascontiguousarray(X5.cpu().numpy().T)
    bt5 = np.ascontiguousarray(dY5.cpu().numpy().T)
    g = dW5f.cpu().numpy()
    bad += int(np.count_nonzero(g[1029].view(np.uint32) !=
                                oracle.gemm(a5[1029:1030], bt5, trans_b=True, fused=True)[0].view(np.uint32)))
    bad += int(np.count_nonzero(g[:, 77].view(np.uint32) !=
                                oracle.gemm(a5, bt5[77:78], trans_b=True, fused=True)[:, 0].view(np.uint32)))
    return {"gemm_fma_sampled_words_differing": bad, "gemm_fma_seconds": round(time.time() - t, 1)}


def verify_in_turn(np, torch, br, state2, digest2, ws, n, aidx, samples, hp, step0, ah_end):
    """The copy updated by the separate calls: every AdamW step of the run
    replayed by the oracle on the sampled elements (the steps', then the
    separate calls'), and the last digest against a fresh hash of the final
    state."""
    import oracle
    t = time.time()
    s_w, s_m, s_v, s_g = samples
    st = np.concatenate([s_w, s_m, s_v]).astype(np.float32)
    for t_ in range(step0, ah_end):  # the steps' updates, then the separate calls'
        oracle.adamw_inplace(st, s_g, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"], t_)
    tidx = torch.from_numpy(aidx).to(state2.device)
    got = np.concatenate([state2[:n][tidx].cpu().numpy(), state2[n:2 * n][tidx].cpu().numpy(),
                          state2[2 * n:][tidx].cpu().numpy()])
    d = torch.empty(32, dtype=torch.uint8, device=state2.device)
    br.repro_state_hash_async(state2, d, ws)
    return {"in_turn_adamw_sampled_words_differing": int(np.count_nonzero(got.view(np.uint32) != st.view(np.uint32))),
            "in_turn_digest_repeats": bool(torch.equal(d, digest2)),
            "in_turn_seconds": round(time.time() - t, 1)}


def verify_bf16(np, torch, br, b_g, b_w, b_m, b_v, b_state, idx, samples, bhp, nsteps):
    """The BF16 step: the device norm against the oracle's over the whole
    gradient, then every step replayed by the oracle on the sampled elements
    (the gradient is the same each step, so each step applied the same clip
    coefficient; the oracle applies it first and runs without the rules)."""
    import oracle
    t = time.time()
    g_bits = b_g.view(torch.int16).cpu().numpy().view(np.uint16)
    norm = oracle.grad_norm(g_bits)
    del g_bits
    st = br.read_step_state(b_state)
    res = {"bf16_norm_matches": bool(np.float32(st["grad_norm"]) == norm),
           "bf16_steps_applied": int(st["step"])}
    coef = np.float32(1.0) / (norm + np.float32(1e-6))
    gc = (oracle.bf16_widen(samples["g"]) * coef).astype(np.float32) if coef < 1 else oracle.bf16_widen(samples["g"])
    w, m, v = samples["w"].copy(), samples["m"].copy(), samples["v"].copy()
    so = oracle.new_step_state()
    hp = {k: bhp[k] for k in ("lr", "beta1", "beta2", "eps", "weight_decay")}
    for _ in range(nsteps):
        oracle.adamw_bf16_step(w, m, v, gc, so, **hp, max_norm=0.0, spike_threshold=0.0)
    tidx = torch.from_numpy(idx).to(b_w.device)
    bad = int(np.count_nonzero(b_w[tidx].view(torch.int16).cpu().numpy().view(np.uint16) != w))
    bad += int(np.count_nonzero(b_m[tidx].cpu().numpy().view(np.uint32) != m.view(np.uint32)))
    bad += int(np.count_nonzero(b_v[tidx].cpu().numpy().view(np.uint32) != v.view(np.uint32)))
    res["bf16_sampled_words_differing"] = bad
    res["bf16_seconds"] = round(time.time() - t, 1)
    return res


def cpu_baseline(np):
    """The oracle timed on a bounded sample of the same step (one host core)."""
    import oracle
    import synth
    # The whole reduce workload and two thirds of the optimizer workload
    # (n = 8e8, a multiple of the 1024-word leaf): 13-15 s of oracle time.
    n_red = synth.REDUCE["n"]
    n_adam = synth.ADAMW["n"] * 2 // 3
    reps = [synth.reduce_replica(r, n_red) for r in range(8)]
    st = np.concatenate([synth.adamw_w(n_adam), synth.adamw_m(n_adam), synth.adamw_v(n_adam)])
    g = synth.adamw_g(n_adam)
    x = synth.gemm_x(rows=16).reshape(16, 2048)
    bt = np.ascontiguousarray(synth.gemm_w().reshape(2048, 8192).T)
    # The weight-gradient shape: 8 output rows of dW = X^T dY (K = 16,384
    # terms per chain), i.e. 8 columns of X against dY, with dY transposed so
    # that the oracle's k loop reads both operands contiguously.
    dw_rows = 8
    xw = np.ascontiguousarray(synth.dw_x().reshape(16384, 2048)[:, :dw_rows].T)
    dyt = np.ascontiguousarray(synth.dw_dy().reshape(16384, 8192).T)
    # One thread on one core: the calling thread is pinned for the timed part.
    try:
        saved = os.sched_getaffinity(0)
        core = min(saved)
        os.sched_setaffinity(0, {core})
    except (AttributeError, OSError):
        saved, core = None, None
    t0 = time.perf_counter()
    oracle.tree_reduce(reps)
    t1 = time.perf_counter()
    oracle.adamw_inplace(st, g, 3e-4, 0.9, 0.999, 1e-8, 0.1, 1000)
    t2 = time.perf_counter()
    oracle.state_hash(st)
    t3 = time.perf_counter()
    oracle.gemm(x, bt, trans_b=True)
    t4 = time.perf_counter()
    oracle.gemm(xw, dyt, trans_b=True)
    t5 = time.perf_counter()
    if saved is not None:
        os.sched_setaffinity(0, saved)
    del xw, dyt
    nbytes = 9 * 4 * n_red + 28 * n_adam + 12 * n_adam
    return {"value": round(nbytes / (t3 - t0) / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "gemm_gflops": round(2 * 16 * 8192 * 2048 / (t4 - t3) / 1e9, 4),
            "gemm_dw_gflops": round(2 * dw_rows * 8192 * 16384 / (t5 - t4) / 1e9, 4),
            "sample": f"the reduce workload (R=8 n={n_red}) and 2/3 of the optimizer workload (adamw + state_hash "
                      f"n={n_adam}); gemm: 16 rows of 8192x2048x8192 and {dw_rows} rows of dW 2048x8192 "
                      f"(K=16384); single-threaded oracle, {t5 - t0:.1f} s",
            "host_cpu": _cpu_model(), "host_threads": os.cpu_count(), "pinned_core": core}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
