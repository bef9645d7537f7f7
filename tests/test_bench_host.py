"""Host logic of bench.py that runs without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    # The library has no multi-GPU path: bench.py measures one GPU and says so
    # (before it imports torch or touches a device).
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 2" in res.stderr
    assert res.stdout == ""


def test_traffic_lines_parse():
    # Every op line of the committed counter summary names a source that
    # exists; traffic is reported only for sources unchanged since.
    sys.path.insert(0, ROOT)
    import bench
    path = os.path.join(ROOT, "profiles", "pmc_traffic_bench_step.md")
    ops = [ln.split()[1] for ln in open(path).read().splitlines() if ln.startswith("traffic ")]
    assert {"tree_reduce", "gemm_fwd", "adamw_state_hash", "gemm_dw"} <= set(ops)
    for ln in open(path).read().splitlines():
        if ln.startswith("traffic "):
            for f in ln.split()[3].split("+"):
                assert os.path.exists(os.path.join(ROOT, "bitwise_reproducible_amd", "csrc", f)), f
    got = bench.recorded_traffic()
    assert set(got) <= set(ops) and all(v > 0 for v in got.values())
