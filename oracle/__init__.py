"""CPU oracle for the reproducible operations (ctypes over ``librepro_oracle.so``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU library never does.  Every function below
only marshals numpy arrays into the C oracle, which holds all the arithmetic
(see ``repro_oracle.c`` for the definitions and their sources on the pages).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librepro_oracle.so")
_lib = None

OP_ADD, OP_SUB, OP_MUL, OP_DIV, OP_SQRT = range(5)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i64, vp, i32, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        lib.oracle_fp32_ops.argtypes = [ctypes.c_int, vp, vp, vp, i64]
        lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, i64, vp, i64, vp, i64]
        lib.oracle_gemm_fma.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, i64, vp, i64, vp, i64]
        lib.oracle_fma.argtypes = [vp, vp, vp, vp, i64]
        lib.oracle_grad_norm.argtypes = [vp, i32, i64, vp]
        lib.oracle_bf16_round.argtypes = [vp, vp, i64]
        lib.oracle_adamw_bf16_step.argtypes = [vp, vp, vp, vp, i32, i64, f32, f32, f32, f32, f32, f32, f32, i32, vp]
        lib.oracle_tree_reduce.argtypes = [vp, i32, i64, vp, i32, vp]
        lib.oracle_replay_reduce.argtypes = [vp, i32, i32, i32, i64, vp]
        lib.oracle_fold_push.argtypes = [vp, i32, vp, i64]
        lib.oracle_fold_result.argtypes = [vp, i32, i64, vp, i32]
        lib.oracle_adamw_scalars.argtypes = [f32, f32, i64, vp]
        lib.oracle_adamw.argtypes = [vp, vp, i64, f32, f32, f32, f32, f32, i64]
        lib.oracle_blake2b.argtypes = [vp, i64, ctypes.c_int, vp, vp]
        lib.oracle_state_hash_leaves.argtypes = [vp, i64, i64, i64, vp]
        lib.oracle_state_hash.argtypes = [vp, i64, vp]
        lib.oracle_state_hash_one_leaf.argtypes = [vp, i64, i64, ctypes.c_int, vp]
        lib.oracle_spec_version.restype = ctypes.c_char_p
        for name in ("oracle_fp32_ops", "oracle_gemm", "oracle_tree_reduce", "oracle_adamw_scalars",
                     "oracle_adamw", "oracle_blake2b", "oracle_state_hash_leaves", "oracle_state_hash",
                     "oracle_state_hash_one_leaf", "oracle_replay_reduce", "oracle_fold_push",
                     "oracle_fold_result"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


class swap_library:
    """Context manager: route every call to another build of the oracle
    (used only by the mutation tests, which compile deliberately broken
    copies of ``repro_oracle.c`` to show the pins catch them)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        _load()
        self.saved = _lib
        _lib = None
        saved_path = globals()["_LIB_PATH"]
        globals()["_LIB_PATH"] = self.path
        try:
            _load()
        finally:
            globals()["_LIB_PATH"] = saved_path
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what}: oracle returned {rc}")


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def spec_version() -> str:
    return _load().oracle_spec_version().decode()


def fp32_op(op: int, a, b=None) -> np.ndarray:
    """One contract operation per element (0 add, 1 sub, 2 mul, 3 div, 4 sqrt)."""
    a = _f32(a)
    b = _f32(a if b is None else b)
    assert a.shape == b.shape
    out = np.empty_like(a)
    _check(_load().oracle_fp32_ops(op, a.ctypes.data, b.ctypes.data, out.ctypes.data, a.size), "fp32_ops")
    return out


def fma(a, b, c) -> np.ndarray:
    """fl(a*b + c) rounded once, under the contract's subnormal rule."""
    a, b, c = _f32(a), _f32(b), _f32(c)
    assert a.shape == b.shape == c.shape
    out = np.empty_like(a)
    _check(_load().oracle_fma(a.ctypes.data, b.ctypes.data, c.ctypes.data, out.ctypes.data, a.size), "fma")
    return out


def gemm(A, B, trans_a: bool = False, trans_b: bool = False, fused: bool = False) -> np.ndarray:
    """C = op(A) @ op(B) with one ascending-k chain per output: unfused
    multiply then add (the pages' convention), or fused when `fused`."""
    A = _f32(A)
    B = _f32(B)
    M, K = (A.shape[1], A.shape[0]) if trans_a else A.shape
    K2, N = (B.shape[1], B.shape[0]) if trans_b else B.shape
    assert K == K2, "inner dimensions differ"
    C = np.empty((M, N), dtype=np.float32)
    lda = A.shape[1] if A.ndim == 2 and A.shape[1] > 0 else 1
    ldb = B.shape[1] if B.ndim == 2 and B.shape[1] > 0 else 1
    fn = _load().oracle_gemm_fma if fused else _load().oracle_gemm
    _check(fn(int(trans_a), int(trans_b), M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb, C.ctypes.data,
              max(N, 1)), "gemm")
    return C


# The optimizer-step record (same field order as the library's).
STEP_STATE = np.dtype([("step", "<i8"), ("skip_left", "<i4"), ("applied", "<i4"), ("beta1_pow", "<f4"),
                       ("beta2_pow", "<f4"), ("grad_norm", "<f4"), ("clip_coef", "<f4")])


def new_step_state() -> np.ndarray:
    """A fresh record: no step applied, nothing to skip (all fields zero)."""
    return np.zeros(1, STEP_STATE)


def _grad_arg(g):
    g = np.ascontiguousarray(g)
    if g.dtype == np.uint16:  # bf16 bit patterns
        return g, 1
    return np.ascontiguousarray(g, np.float32), 0


def grad_norm(g, return_sumsq: bool = False):
    """Pre-clip global l2 norm: sqrt of the TreeFold of the squares (g float32,
    or uint16 bf16 patterns); with return_sumsq, (norm, S)."""
    g, dt = _grad_arg(g)
    out = np.zeros(2, np.float32)
    _check(_load().oracle_grad_norm(g.ctypes.data, dt, g.size, out.ctypes.data), "grad_norm")
    return (out[0], out[1]) if return_sumsq else out[0]


def bf16_round(x) -> np.ndarray:
    """binary32 -> bf16 bit patterns (uint16), nearest-even."""
    x = _f32(x)
    out = np.empty(x.shape, np.uint16)
    _check(_load().oracle_bf16_round(x.ctypes.data, out.ctypes.data, x.size), "bf16_round")
    return out


def bf16_widen(h) -> np.ndarray:
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def adamw_bf16_step(w, m, v, g, state, lr, beta1, beta2, eps, weight_decay, max_norm=1.0, spike_threshold=5.0,
                    skip_steps=5) -> None:
    """One optimizer step in place: w uint16 (bf16), m and v float32, g float32 or uint16 (bf16)."""
    assert w.dtype == np.uint16 and m.dtype == np.float32 and v.dtype == np.float32 and state.dtype == STEP_STATE
    assert w.flags.c_contiguous and m.flags.c_contiguous and v.flags.c_contiguous
    g, dt = _grad_arg(g)
    n = w.size
    assert m.size == n and v.size == n and g.size == n
    _check(_load().oracle_adamw_bf16_step(w.ctypes.data, m.ctypes.data, v.ctypes.data, g.ctypes.data, dt, n, lr,
                                          beta1, beta2, eps, weight_decay, max_norm, spike_threshold, skip_steps,
                                          state.ctypes.data), "adamw_bf16_step")


def tree_reduce(replicas, average: bool = True, return_resident: bool = False):
    reps = [_f32(r).reshape(-1) for r in replicas]
    R = len(reps)
    n = reps[0].size if R else 0
    assert all(r.size == n for r in reps)
    ptrs = (ctypes.c_void_p * max(R, 1))(*[r.ctypes.data for r in reps])
    out = np.empty(n, dtype=np.float32)
    resident = ctypes.c_int32(0)
    _check(_load().oracle_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), R, n, out.ctypes.data,
                                      int(average), ctypes.addressof(resident)), "tree_reduce")
    return (out, resident.value) if return_resident else out


def adamw_scalars(beta1: float, beta2: float, step: int) -> np.ndarray:
    """The host scalars (c1, c2, r1, r2) as binary32."""
    out = np.zeros(4, dtype=np.float32)
    _check(_load().oracle_adamw_scalars(beta1, beta2, step, out.ctypes.data), "adamw_scalars")
    return out


def adamw(state, grad, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float,
          step: int) -> np.ndarray:
    """Returns the updated flat [w | m | v] state (the input is not modified)."""
    st = np.array(state, dtype=np.float32, copy=True).reshape(-1)
    g = _f32(grad).reshape(-1)
    n = g.size
    assert st.size == 3 * n
    _check(_load().oracle_adamw(st.ctypes.data, g.ctypes.data, n, lr, beta1, beta2, eps, weight_decay,
                                step), "adamw")
    return st


def adamw_inplace(state: np.ndarray, grad: np.ndarray, lr, beta1, beta2, eps, weight_decay, step):
    assert state.dtype == np.float32 and state.flags.c_contiguous
    g = _f32(grad).reshape(-1)
    assert state.size == 3 * g.size
    _check(_load().oracle_adamw(state.ctypes.data, g.ctypes.data, g.size, lr, beta1, beta2, eps,
                                weight_decay, step), "adamw")


def blake2b(data: bytes, digest_size: int = 64, person: bytes = b"") -> bytes:
    buf = np.frombuffer(bytes(data), dtype=np.uint8) if data else np.zeros(1, dtype=np.uint8)
    p = np.zeros(16, dtype=np.uint8)
    p[:len(person)] = np.frombuffer(person, dtype=np.uint8)
    out = np.zeros(64, dtype=np.uint8)
    _check(_load().oracle_blake2b(buf.ctypes.data, len(data), digest_size, p.ctypes.data, out.ctypes.data),
           "blake2b")
    return out[:digest_size].tobytes()


def state_hash(words) -> bytes:
    w = _f32(words).reshape(-1)
    out = np.zeros(32, dtype=np.uint8)
    ptr = w.ctypes.data if w.size else np.zeros(1, np.float32).ctypes.data
    _check(_load().oracle_state_hash(ptr, w.size, out.ctypes.data), "state_hash")
    return out.tobytes()


def state_hash_leaves(words, leaf0: int, count: int) -> np.ndarray:
    w = _f32(words).reshape(-1)
    out = np.zeros((count, 32), dtype=np.uint8)
    ptr = w.ctypes.data if w.size else np.zeros(1, np.float32).ctypes.data
    _check(_load().oracle_state_hash_leaves(ptr, w.size, leaf0, count, out.ctypes.data), "state_hash_leaves")
    return out


def state_hash_one_leaf(words, leaf: int, last: bool) -> bytes:
    """Digest of one leaf (at most 1024 words) placed at node offset `leaf`."""
    w = _f32(words).reshape(-1)
    out = np.zeros(32, dtype=np.uint8)
    ptr = w.ctypes.data if w.size else np.zeros(1, np.float32).ctypes.data
    _check(_load().oracle_state_hash_one_leaf(ptr, w.size, leaf, int(last), out.ctypes.data), "state_hash_one_leaf")
    return out.tobytes()


def replay_reduce(grads, dp_replicate: int, dp_shard: int, accum: int) -> np.ndarray:
    """Algorithm 1's reduction: grads in mesh order, rank-major then microbatch."""
    bufs = [_f32(g).reshape(-1) for g in grads]
    assert len(bufs) == dp_replicate * dp_shard * accum
    n = bufs[0].size
    assert all(b.size == n for b in bufs)
    ptrs = (ctypes.c_void_p * len(bufs))(*[b.ctypes.data for b in bufs])
    out = np.empty(n, dtype=np.float32)
    _check(_load().oracle_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), dp_replicate, dp_shard, accum, n,
                                        out.ctypes.data), "replay_reduce")
    return out


def fold_push(slots, pushed: int, part) -> None:
    """Streaming TreeFold push into a list of numpy level slots (modified in place)."""
    p = _f32(part).reshape(-1)
    for sl in slots:
        assert sl.dtype == np.float32 and sl.flags.c_contiguous and sl.size == p.size
    ptrs = (ctypes.c_void_p * len(slots))(*[sl.ctypes.data for sl in slots])
    _check(_load().oracle_fold_push(ctypes.cast(ptrs, ctypes.c_void_p), pushed, p.ctypes.data, p.size), "fold_push")


def fold_result(slots, pushed: int, divisor: int = 0) -> np.ndarray:
    n = slots[0].size
    ptrs = (ctypes.c_void_p * len(slots))(*[sl.ctypes.data for sl in slots])
    out = np.empty(n, dtype=np.float32)
    _check(_load().oracle_fold_result(ctypes.cast(ptrs, ctypes.c_void_p), pushed, n, out.ctypes.data, divisor),
           "fold_result")
    return out
