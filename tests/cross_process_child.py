"""Child process for the cross-process determinism test.

Default mode: runs the tiny chained workload (GEMM, TreeFold, AdamW, state
hash), the full gradient-reduction workload, and small cases of the audit
replay, the fused GEMM convention (both units), the fused AdamW + hash and the
BF16 optimizer step, ten times each in a fresh process, and prints one JSON
line of SHA-256 digests of the output words.

``--full``: the four full-size workloads, ten runs each in this process, every
output reduced on the GPU to its 32-byte state hash (repro_state_hash):
TreeFold over 8 x 16,777,216; the forward GEMM 8192 x 2048 x 8192; the weight
gradient X^T dY with K = 16,384; the fused AdamW + state hash on the
1.2e9-parameter [w | m | v] from the same initial state each run (the fused
call's own digest and a separate state hash of the updated state).  Prints one
JSON line of hex digests per run.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import bitwise_reproducible_amd as br  # noqa: E402
import synth  # noqa: E402


def sha(t) -> str:
    return hashlib.sha256(t.detach().cpu().numpy().tobytes()).hexdigest()


REPLAY_LAYOUT = (3, 2, 2)
AH_HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=5)
BF16_HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0, spike_threshold=5.0,
               skip_steps=5)


def replay_inputs():
    return [synth.generate(4099, synth.OUTLIER_SCALED, synth.tid(9, b), 1e-3, 0.01, 1e4) for b in range(12)]


def adamw_hash_inputs():
    n = 64 * 1024
    st = np.concatenate([synth.generate(n, synth.NORMAL, synth.tid(9, 0x20), 0.02),
                         synth.generate(n, synth.NORMAL, synth.tid(9, 0x21), 1e-4),
                         synth.generate(n, synth.HALF_NORMAL, synth.tid(9, 0x22), 1e-6)])
    return st, synth.generate(n, synth.NORMAL, synth.tid(9, 0x23), 1e-3)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def bf16_inputs():
    n = 5003
    w = _bf16_bits(synth.generate(n, synth.NORMAL, synth.tid(9, 0x30), 0.02))
    m = synth.generate(n, synth.NORMAL, synth.tid(9, 0x31), 1e-4)
    v = synth.generate(n, synth.HALF_NORMAL, synth.tid(9, 0x32), 1e-6)
    g = _bf16_bits(synth.generate(n, synth.NORMAL, synth.tid(9, 0x33), 0.03))  # norm ~2: clipped
    return w, m, v, g


def main():
    dev = torch.device("cuda:0")
    cfg = synth.TINY
    out = {"pid": os.getpid()}
    a, b = synth.tiny_gemm_inputs()
    da, db = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    reps = [torch.from_numpy(synth.tiny_replica(r)).to(dev) for r in range(cfg["R"])]
    n = cfg["n"]
    state0 = torch.from_numpy(np.concatenate([synth.tiny_adamw_weights(n), np.zeros(2 * n, np.float32)])).to(dev)
    hp = (cfg["lr"], cfg["beta1"], cfg["beta2"], cfg["eps"], cfg["wd"], cfg["step"])
    big = [torch.from_numpy(synth.reduce_replica(r)).to(dev) for r in range(synth.REDUCE["R"])]
    grads = [torch.from_numpy(x).to(dev) for x in replay_inputs()]
    ah_state0, ah_g = (torch.from_numpy(x).to(dev) for x in adamw_hash_inputs())
    ah_ws = br.hash_workspace(ah_state0.numel())
    w0, m0, v0, gb = bf16_inputs()
    runs = []
    for _ in range(10):
        g = br.repro_tree_reduce(reps)
        st = state0.clone()
        br.repro_adamw(st, g, *hp)
        r = {"gemm": sha(br.repro_gemm(da, db)), "reduce": sha(g), "adamw": sha(st),
             "state_hash": br.repro_state_hash(st).hex(), "reduce_workload": sha(br.repro_tree_reduce(big)),
             "replay": sha(br.repro_replay_reduce(grads, *REPLAY_LAYOUT)),
             "gemm_fma0": sha(br.repro_gemm_fma(da, db, variant=0)),
             "gemm_fma1": sha(br.repro_gemm_fma(da, db, variant=1))}
        ah = ah_state0.clone()
        dg = torch.empty(32, dtype=torch.uint8, device=dev)
        br.repro_adamw_hash(ah, ah_g, dg, ah_ws, **AH_HP)
        r["adamw_hash_state"] = sha(ah)
        r["adamw_hash_digest"] = bytes(dg.cpu().numpy()).hex()
        w = torch.from_numpy(w0.view(np.int16)).to(dev).view(torch.bfloat16)
        m, v = torch.from_numpy(m0).to(dev), torch.from_numpy(v0).to(dev)
        gdev = torch.from_numpy(gb.view(np.int16)).to(dev).view(torch.bfloat16)
        sdev = br.new_step_state(dev)
        for _k in range(3):
            br.repro_adamw_bf16_step(w, m, v, gdev, sdev, **BF16_HP)
        r["bf16_w"] = sha(w.view(torch.int16))
        r["bf16_m"] = sha(m)
        runs.append(r)
    out["runs"] = runs
    print(json.dumps(out), flush=True)


def _digest(t, ws) -> str:
    return br.repro_state_hash(t.reshape(-1), ws).hex()


def main_full():
    dev = torch.device("cuda:0")
    out = {"pid": os.getpid()}
    runs = [dict() for _ in range(10)]

    def stage(name):
        print(f"full-size stage: {name}", file=sys.stderr, flush=True)

    stage("tree reduce")
    reps = [torch.from_numpy(synth.reduce_replica(r)).to(dev) for r in range(synth.REDUCE["R"])]
    ws = br.hash_workspace(synth.REDUCE["n"], dev)
    for r in runs:
        r["reduce"] = _digest(br.repro_tree_reduce(reps), ws)
    del reps, ws
    stage("forward gemm")
    cfg = synth.GEMM
    X = torch.from_numpy(synth.gemm_x()).to(dev).view(cfg["M"], cfg["K"])
    W = torch.from_numpy(synth.gemm_w()).to(dev).view(cfg["K"], cfg["N"])
    Y = torch.empty(cfg["M"], cfg["N"], dtype=torch.float32, device=dev)
    ws = br.hash_workspace(Y.numel(), dev)
    for r in runs:
        Y.fill_(7.0)
        br.repro_gemm(X, W, out=Y)
        r["gemm_fwd"] = _digest(Y, ws)
    del X, W, Y, ws
    stage("weight gradient gemm")
    cfg = synth.DW
    Xd = torch.from_numpy(synth.dw_x()).to(dev).view(cfg["K"], cfg["M"])
    dY = torch.from_numpy(synth.dw_dy()).to(dev).view(cfg["K"], cfg["N"])
    dW = torch.empty(cfg["M"], cfg["N"], dtype=torch.float32, device=dev)
    ws = br.hash_workspace(dW.numel(), dev)
    for r in runs:
        dW.fill_(7.0)
        br.repro_gemm(Xd, dY, trans_a=True, out=dW)
        r["gemm_dw"] = _digest(dW, ws)
    del Xd, dY, dW, ws
    stage("fused adamw + state hash, n = 1.2e9")
    cfg = synth.ADAMW
    n = cfg["n"]
    host = np.empty(3 * n, np.float32)
    synth.adamw_w(n, out=host[:n])
    synth.adamw_m(n, out=host[n:2 * n])
    synth.adamw_v(n, out=host[2 * n:])
    state0 = torch.from_numpy(host).to(dev)
    del host
    g = torch.from_numpy(synth.adamw_g()).to(dev)
    st = torch.empty_like(state0)
    ws = br.hash_workspace(3 * n, dev)
    dg = torch.empty(32, dtype=torch.uint8, device=dev)
    hp = dict(lr=cfg["lr"], beta1=cfg["beta1"], beta2=cfg["beta2"], eps=cfg["eps"], weight_decay=cfg["wd"],
              step=cfg["step"])
    for r in runs:
        st.copy_(state0)
        br.repro_adamw_hash(st, g, dg, ws, **hp)
        r["adamw_hash_digest"] = bytes(dg.cpu().numpy()).hex()
        r["adamw_state"] = _digest(st, ws)
    stage("done")
    out["runs"] = runs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main_full() if "--full" in sys.argv[1:] else main()
