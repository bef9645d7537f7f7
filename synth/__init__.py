"""Seeded synthetic inputs for the five reproducible-ops workloads.

Holds none of the operations' arithmetic: it only produces input tensors.
The values come from ``libsynth.so`` (Philox4x64-10 + Box-Muller in binary64,
rounded once to binary32; see ``synth_gen.c``).  A value is a pure function of
(seed, tensor id, element index), so any slice can be regenerated on its own.

Workload recipes (sizes and distributions as the workload table states; the
second argument of N(., .) is a standard deviation, as the OPEN-1B paper uses
it for its initialisation in section 3.1):

* tiny    - GEMM 64x64x64, A,B ~ N(0,1); tree reduce R=4, n=65,536, each
            N(0,1e-3) with 1% of entries scaled x1e4; AdamW on n=65,536 with
            w ~ N(0,0.02), m = v = 0, grad = the reduce output, step 1.
* reduce  - R=8 replicas of n=16,777,216, N(0,1e-3) with 0.1% of entries
            replaced by N(0,10).
* gemm    - X[8192x2048] ~ N(0,1) times W[2048x8192] ~ N(0,0.02).
* adamw   - n=1.2e9: w ~ N(0,0.02), m ~ N(0,1e-4), v = |N(0,1e-6)|,
            g ~ N(0,1e-3); step 1000, lr 3e-4, wd 0.1.
* dw      - dW = X^T dY with X[16384x2048], dY[16384x8192], both 1e-2 * t(3).
* replay  - the audit replay of one step's reduction at the OPEN-1B main-phase
            layout: 6 replicas x 8 shards x 6 microbatches = 288 gradient
            buffers of an n=8,388,608 slice, each N(0,1e-3) with 0.1% of
            entries replaced by N(0,10).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

SEED = 42  # the run seed of the OPEN-1B recipe (section 3.2)

NORMAL, HALF_NORMAL, OUTLIER_SCALED, OUTLIER_REPLACE, STUDENT_T3, UNIFORM = range(6)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                   ctypes.c_double, ctypes.c_double, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_int]
        lib.synth_philox4x64_10.restype = None
        lib.synth_philox4x64_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def philox4x64_10(counter, key):
    """One Philox4x64-10 block (four uint64) for a counter (4 words) and key (2 words)."""
    lib = _load()
    c = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib.synth_philox4x64_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def fill_into(ptr: int, n: int, kind: int, tid: int, std: float, p1: float = 0.0, p2: float = 0.0,
              offset: int = 0, seed: int = SEED, threads: int | None = None) -> None:
    """Write elements [offset, offset+n) of a stream into host memory at ``ptr``."""
    lib = _load()
    rc = lib.synth_fill(int(kind), int(seed), int(tid), float(std), float(p1), float(p2), int(offset),
                        int(n), ctypes.c_void_p(int(ptr)), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("synth_fill rejected its arguments")


def generate(n: int, kind: int, tid: int, std: float, p1: float = 0.0, p2: float = 0.0,
             offset: int = 0, seed: int = SEED, threads: int | None = None, out=None) -> np.ndarray:
    if out is None:
        out = np.empty(int(n), dtype=np.float32)
    assert out.dtype == np.float32 and out.flags.c_contiguous and out.size == n
    fill_into(out.ctypes.data, n, kind, tid, std, p1, p2, offset, seed, threads)
    return out


# --------------------------------------------------------------------------
# Tensor ids: config number in the high byte, tensor index in the low byte.
def tid(config: int, index: int) -> int:
    return (config << 8) | index


# Workload definitions -------------------------------------------------------
TINY = dict(gemm=(64, 64, 64), R=4, n=65536, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.1, step=1)
REDUCE = dict(R=8, n=16_777_216)
GEMM = dict(M=8192, N=8192, K=2048)
ADAMW = dict(n=1_200_000_000, lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.1, step=1000)
DW = dict(M=2048, N=8192, K=16384)
REPLAY = dict(dp_replicate=6, dp_shard=8, accum=6, n=8_388_608)


def tiny_gemm_inputs(M=64, N=64, K=64):
    a = generate(M * K, NORMAL, tid(1, 0x00), 1.0).reshape(M, K)
    b = generate(K * N, NORMAL, tid(1, 0x01), 1.0).reshape(K, N)
    return a, b


def tiny_replica(r: int, n: int = 65536, offset: int = 0, out=None):
    return generate(n, OUTLIER_SCALED, tid(1, 0x10 + r), 1e-3, 0.01, 1e4, offset=offset, out=out)


def tiny_adamw_weights(n: int = 65536, offset: int = 0, out=None):
    return generate(n, NORMAL, tid(1, 0x20), 0.02, offset=offset, out=out)


def reduce_replica(r: int, n: int = REDUCE["n"], offset: int = 0, out=None):
    return generate(n, OUTLIER_REPLACE, tid(2, 0x10 + r), 1e-3, 0.001, 10.0, offset=offset, out=out)


def gemm_x(rows=GEMM["M"], cols=GEMM["K"], row0=0, out=None):
    """Rows [row0, row0+rows) of X[8192 x 2048] ~ N(0,1), row-major."""
    full_cols = GEMM["K"]
    assert cols == full_cols
    return generate(rows * cols, NORMAL, tid(3, 0x00), 1.0, offset=row0 * full_cols, out=out)


def gemm_w(rows=GEMM["K"], cols=GEMM["N"], row0=0, out=None):
    full_cols = GEMM["N"]
    assert cols == full_cols
    return generate(rows * cols, NORMAL, tid(3, 0x01), 0.02, offset=row0 * full_cols, out=out)


def adamw_w(n=ADAMW["n"], offset=0, out=None):
    return generate(n, NORMAL, tid(4, 0x00), 0.02, offset=offset, out=out)


def adamw_m(n=ADAMW["n"], offset=0, out=None):
    return generate(n, NORMAL, tid(4, 0x01), 1e-4, offset=offset, out=out)


def adamw_v(n=ADAMW["n"], offset=0, out=None):
    return generate(n, HALF_NORMAL, tid(4, 0x02), 1e-6, offset=offset, out=out)


def adamw_g(n=ADAMW["n"], offset=0, out=None):
    return generate(n, NORMAL, tid(4, 0x03), 1e-3, offset=offset, out=out)


def dw_x(rows=DW["K"], row0=0, out=None):
    """Rows [row0, row0+rows) of X[16384 x 2048] ~ 1e-2 t(3), row-major."""
    cols = DW["M"]
    return generate(rows * cols, STUDENT_T3, tid(5, 0x00), 1e-2, offset=row0 * cols, out=out)


def dw_dy(rows=DW["K"], row0=0, out=None):
    cols = DW["N"]
    return generate(rows * cols, STUDENT_T3, tid(5, 0x01), 1e-2, offset=row0 * cols, out=out)


def replay_grad(b: int, n: int = REPLAY["n"], offset: int = 0, out=None):
    """Microbatch gradient buffer b (mesh order, rank-major) of the replay workload.

    Its 288 tensor ids sit above the one-byte index range of the other
    workloads: 0x60000 + b."""
    return generate(n, OUTLIER_REPLACE, (6 << 16) | b, 1e-3, 0.001, 10.0, offset=offset, out=out)
