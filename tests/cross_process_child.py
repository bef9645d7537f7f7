"""Child process for the cross-process determinism test.

Runs the tiny chained workload (GEMM, TreeFold, AdamW, state hash) and the
full gradient-reduction workload ten times each in a fresh process and prints
one JSON line of SHA-256 digests of the output words.
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
    runs = []
    for _ in range(10):
        g = br.repro_tree_reduce(reps)
        st = state0.clone()
        br.repro_adamw(st, g, *hp)
        runs.append({"gemm": sha(br.repro_gemm(da, db)), "reduce": sha(g), "adamw": sha(st),
                     "state_hash": br.repro_state_hash(st).hex(), "reduce_workload": sha(br.repro_tree_reduce(big))})
    out["runs"] = runs
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
