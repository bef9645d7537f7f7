"""Resume on the GPU from a checkpoint record equals a run that never stopped.

The checkpoint page's flat record [int32 step][int32 n][w | m | v] (saving the
moments is what makes a resumed run bit-equivalent to an uninterrupted one)
and OPEN-1B section 3.4 (restarts from checkpoints, validated by hashing).
Child processes run repro_adamw_hash steps on the GPU: one runs steps 1..12
without stopping; another writes the record after every step and exits
right after step 5 is recorded (its GPU work finished); a third
resumes from that record in a fresh process.  The resumed state and the
library's state hash equal the uninterrupted run's and the oracle's.

This module is named to run before the GPU tests that initialise the GPU in
the test process itself: the test process here only starts children.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle
from checkpoint_record import read_record

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CHILD = os.path.join(HERE, "resume_child.py")
STEPS = 12


def _run(*args):
    res = subprocess.run([sys.executable, CHILD, *args], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


def test_gpu_resume_from_record_matches_uninterrupted_run(tmp_path):
    print("uninterrupted gpu child", flush=True)
    whole = json.loads(_run("gpu", "0", str(STEPS), "-", "-").strip().splitlines()[-1])
    rec = str(tmp_path / "ckpt.bin")
    print("gpu child stopping after step 5", flush=True)
    out = _run("gpu", "0", str(STEPS), "-", rec, "--stop-after", "5")
    assert out.strip().splitlines()[-1] == "step 5"  # it exited right after the record of step 5
    assert read_record(rec)[0] == 5
    print("resumed gpu child", flush=True)
    resumed = json.loads(_run("gpu", "5", str(STEPS), rec, "-").strip().splitlines()[-1])
    assert resumed["pid"] != whole["pid"]
    assert resumed["state_sha"] == whole["state_sha"]
    assert resumed["digest"] == whole["digest"]
    # ...and both are the oracle's.
    ref = json.loads(_run("oracle", "0", str(STEPS), "-", "-").strip().splitlines()[-1])
    assert whole["state_sha"] == ref["state_sha"] and whole["digest"] == ref["digest"]
    assert oracle.spec_version() == "repro-spec-1"
