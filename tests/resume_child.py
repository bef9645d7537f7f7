"""Child process for the resume tests: AdamW steps on the flat state, with a
checkpoint record written after chosen steps.

    python resume_child.py (oracle|gpu) START STOP RECORD_IN|- RECORD_OUT|- [--stop-after K] [--hang-after K]

Steps START+1 .. STOP are applied (the state comes from RECORD_IN, whose step
must equal START, or is the seeded initial state when RECORD_IN is '-' and
START is 0).  Each step t uses its own seeded gradient.  After every step the
record is written to RECORD_OUT (when given) and a line "step t" is printed.
--stop-after K ends the process right after step K is recorded (the GPU work
of the step has finished first); --hang-after K makes the oracle child wait
after step K until it is killed (CPU only).  At the end one JSON line gives
the state's SHA-256 and the state hash.
"""
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import numpy as np  # noqa: E402

import synth  # noqa: E402
from checkpoint_record import read_record, write_record  # noqa: E402

N = 1024 * 24
HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def initial_state():
    return np.concatenate([synth.generate(N, synth.NORMAL, synth.tid(0x0B, 0), 0.02),
                           synth.generate(N, synth.NORMAL, synth.tid(0x0B, 1), 1e-4),
                           np.abs(synth.generate(N, synth.NORMAL, synth.tid(0x0B, 2), 1e-6))]).astype(np.float32)


def grad_for(step: int):
    return synth.generate(N, synth.NORMAL, synth.tid(0x0C, step & 0xFF), 1e-3, offset=N * (step >> 8))


def main():
    mode, start, stop, rin, rout = sys.argv[1], int(sys.argv[2]), int(sys.argv[3]), sys.argv[4], sys.argv[5]
    stop_after = int(sys.argv[sys.argv.index("--stop-after") + 1]) if "--stop-after" in sys.argv else None
    hang_after = int(sys.argv[sys.argv.index("--hang-after") + 1]) if "--hang-after" in sys.argv else None
    if rin == "-":
        assert start == 0
        state = initial_state()
    else:
        step0, state = read_record(rin)
        assert step0 == start, (step0, start)
    if mode == "gpu":
        import torch
        import bitwise_reproducible_amd as br
        dev = torch.device("cuda:0")
        st = torch.from_numpy(state.copy()).to(dev)
        digest = torch.empty(32, dtype=torch.uint8, device=dev)
        ws = br.hash_workspace(3 * N, dev)
    else:
        import oracle
    for t in range(start + 1, stop + 1):
        g = grad_for(t)
        if mode == "gpu":
            br.repro_adamw_hash(st, torch.from_numpy(g).to(dev), digest, ws, step=t, **HP)
            torch.cuda.synchronize()
            state = st.cpu().numpy()
        else:
            oracle.adamw_inplace(state, g, step=t, **HP)
        if rout != "-":
            write_record(rout, t, state)
        print(f"step {t}", flush=True)
        if stop_after is not None and t == stop_after:
            sys.exit(0)  # end here, after the record is on disk and the step's GPU work has finished
        if hang_after is not None and t == hang_after:
            while True:
                time.sleep(1)
    out = {"pid": os.getpid(), "step": stop, "state_sha": hashlib.sha256(state.tobytes()).hexdigest()}
    if mode == "gpu":
        out["digest"] = bytes(digest.cpu().numpy()).hex()
    else:
        out["digest"] = oracle.state_hash(state).hex()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
