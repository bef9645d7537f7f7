"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host only).

Builds the oracle source together with tests/oracle_sanitize_driver.c, which
calls every oracle entry point on small and edge-case inputs held in
exactly-sized heap buffers, and runs it: any out-of-bounds access, use after
free, leak or undefined integer operation ends the run with an error.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_sanitizers():
    flags = [f for f in oracle_build.FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["gcc", *flags, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", oracle_build.SRC, os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", exe,
               "-lm"]
        subprocess.run(cmd, check=True, capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert res.returncode == 0, res.stderr[-3000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_a_planted_overrun_is_caught():
    # One element past the end in oracle_fma: the sanitized run must fail.
    src = open(oracle_build.SRC).read()
    find = "for (int64_t i = 0; i < n; ++i) out[i] = f_fma(a[i], b[i], c[i]);"
    assert find in src
    flags = [f for f in oracle_build.FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        mutated = os.path.join(d, "oracle_mutated.c")
        open(mutated, "w").write(src.replace(find, find.replace("i < n", "i <= n"), 1))
        exe = os.path.join(d, "oracle_sanitized")
        subprocess.run(["gcc", *flags, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", mutated,
                        os.path.join(HERE, "oracle_sanitize_driver.c"), "-o", exe, "-lm"], check=True,
                       capture_output=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
        res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr
