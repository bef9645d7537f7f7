"""The C-ABI library loads, exports every declared symbol, and checks its
arguments on the host (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re
import sys

import pytest

import bitwise_reproducible_amd as br
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "repro.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(repro_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = br.library()
    names = _declared_functions()
    assert "repro_gemm" in names and "repro_state_hash" in names and len(names) >= 11
    for name in names:
        assert hasattr(lib, name), name


def test_spec_version_matches_the_oracle():
    assert br.spec_version() == "repro-spec-1" == oracle.spec_version()
    assert br.strerror(0) == "ok"
    assert "workspace" in br.strerror(-4)


def test_host_side_argument_checks():
    lib = br.library()
    null = None
    # Negative sizes, bad flags, bad R, bad step: rejected before any launch.
    assert lib.repro_gemm(0, 0, -1, 1, 1, null, 1, null, 1, null, 1, null) == -1
    assert lib.repro_gemm(3, 0, 1, 1, 1, null, 1, null, 1, null, 1, null) == -1
    assert lib.repro_gemm(0, 0, 0, 5, 5, null, 1, null, 1, null, 1, null) == 0  # M == 0: nothing to do
    assert lib.repro_gemm_variant(0, 0, 1, 1, 1, null, 1, null, 1, null, 1, 9, null) == -1
    assert lib.repro_tree_reduce(null, 2, 10, null, 1, null) == -1
    ptrs = (ctypes.c_void_p * 1)(16)
    assert lib.repro_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 65, 10, 16, 1, null) == -1
    assert lib.repro_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 1, 0, null, 1, null) == 0  # n == 0
    assert lib.repro_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 1, 4, 18, 1, null) == -2  # misaligned out
    assert lib.repro_adamw(16, 16, 4, 1e-3, 0.9, 0.999, 1e-8, 0.1, 0, null) == -1
    assert lib.repro_adamw(null, null, 0, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1, null) == 0
    assert lib.repro_fp32_ops(7, 16, 16, 16, 4, null) == -1
    assert lib.repro_state_hash(16, -1, 16, 1 << 20, 16, null) == -1
    assert lib.repro_state_hash(16, 1024, 16, 0, 16, null) == -4  # workspace too small
    # Word counts whose byte count would leave int64 are refused, not wrapped.
    assert lib.repro_state_hash(16, 2**62, 16, 2**40, 16, null) == -1
    assert br.library().repro_state_hash_workspace_bytes(2**62) == -1
    assert lib.repro_adamw_hash(16, 16, 2**61, 1e-3, 0.9, 0.999, 1e-8, 0.1, 1, 16, 2**40, 16, 0, null) == -1
    # Replay: buffer counts whose product would wrap int64 (64 * 2^31-1 * 2^31-1)
    # or exceed the buffer limit are refused before the pointer array is read.
    big = 2**31 - 1
    assert lib.repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 64, big, big, 4, 16, null) == -1
    assert lib.repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 1, 1 << 30, 1 << 28, 4, 16, null) == -1
    assert lib.repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), 2, 1, 193, 4, 16, null) == -1


def _plan_bytes(n_words):
    nbytes = 4 * n_words
    count = max(1, -(-nbytes // 4096))
    total, levels = 0, 0
    while True:
        total += -(-count * 32 // 256) * 256
        levels += 1
        if count == 1 and levels >= 2:
            return total
        count = -(-count // 16)


@pytest.mark.parametrize("n", [0, 1, 1024, 1025, 16 * 1024 + 1, 3 * 1_200_000_000])
def test_hash_workspace_size(n):
    assert br.repro_state_hash_workspace_bytes(n) == _plan_bytes(n)


def test_product_path_has_no_oracle_or_fallback():
    # The package never imports the oracle and has no CPU path: its only
    # compute entry points call into librepro.so.
    pkg_dir = os.path.dirname(br.__file__)
    for dirpath, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "repro_oracle" not in text, f
    assert "oracle" not in sys.modules["bitwise_reproducible_amd"].__dict__


def test_issue_rate_library_exports_its_streams():
    # The measurement library behind the ALU bounds (bench.py --valu-rates):
    # its stream table and entry points load without a GPU.
    path = os.path.join(ROOT, "bitwise_reproducible_amd", "libvalu_rates.so")
    lib = ctypes.CDLL(path)
    for name in ("valu_rates_count", "valu_rates_name", "valu_rates_run", "valu_rates_coissue"):
        assert hasattr(lib, name), name
    lib.valu_rates_name.restype = ctypes.c_char_p
    count = lib.valu_rates_count()
    names = [lib.valu_rates_name(s).decode() for s in range(count)]
    assert count == 14 and len(set(names)) == count
    assert lib.valu_rates_name(count) is None and lib.valu_rates_name(-1) is None
    # Argument checks return before any device call.
    res = (ctypes.c_double * 3)()
    lib.valu_rates_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    lib.valu_rates_coissue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    assert lib.valu_rates_run(count, 2, 10, res) == -1
    assert lib.valu_rates_run(0, 9, 10, res) == -1
    assert lib.valu_rates_coissue(2, 10, 10, res) == -1
    assert lib.valu_rates_coissue(0, 0, 10, res) == -1
