"""Resume from a checkpoint record equals a run that never stopped (CPU oracle).

The checkpoint page: saving w, m and v together makes a resumed run
bit-equivalent to one that never stopped; OPEN-1B section 3.4 restarts its run
from checkpoints and validates the restarts by hashing repeated steps.  Here a
child process applies oracle AdamW steps, writing the flat record
[int32 step][int32 n][w | m | v] after each, and is killed (SIGKILL) while it
waits after step 5; a fresh process resumes from the record and must reach
the same state hash as an uninterrupted run.  Dropping the moments from the
record must change the result (the check can fail).
"""
import json
import os
import signal
import subprocess
import sys

import numpy as np

from checkpoint_record import read_record, write_record

HERE = os.path.dirname(os.path.abspath(__file__))
CHILD = os.path.join(HERE, "resume_child.py")
STEPS = 12


def _run(*args):
    res = subprocess.run([sys.executable, CHILD, *args], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    return json.loads(res.stdout.strip().splitlines()[-1])


def test_record_round_trip(tmp_path):
    p = str(tmp_path / "r.bin")
    st = np.arange(3 * 7, dtype=np.float32) * np.float32(0.25)
    write_record(p, 41, st)
    assert os.path.getsize(p) == 8 + 12 * 7
    step, back = read_record(p)
    assert step == 41 and np.array_equal(back.view(np.uint32), st.view(np.uint32))


def test_killed_process_resumes_bit_for_bit(tmp_path):
    whole = _run("oracle", "0", str(STEPS), "-", "-")
    rec = str(tmp_path / "ckpt.bin")
    proc = subprocess.Popen([sys.executable, CHILD, "oracle", "0", str(STEPS), "-", rec, "--hang-after", "5"],
                            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    try:
        for line in proc.stdout:
            if line.strip() == "step 5":
                break
        else:
            raise AssertionError("the child ended before step 5: " + proc.stderr.read()[-2000:])
        proc.send_signal(signal.SIGKILL)
    finally:
        proc.wait(timeout=60)
    assert proc.returncode == -signal.SIGKILL
    step, _ = read_record(rec)
    assert step == 5
    resumed = _run("oracle", "5", str(STEPS), rec, "-")
    assert resumed["pid"] != whole["pid"]
    assert resumed["state_sha"] == whole["state_sha"] and resumed["digest"] == whole["digest"]
    # Without the moments (m = v = 0 in the record) the resumed run differs.
    _, st = read_record(rec)
    n = st.size // 3
    st[n:] = 0
    bad = str(tmp_path / "no_moments.bin")
    write_record(bad, 5, st)
    assert _run("oracle", "5", str(STEPS), bad, "-")["digest"] != whole["digest"]
