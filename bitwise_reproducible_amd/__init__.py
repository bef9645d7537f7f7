"""Python binding of librepro.so: bitwise-reproducible training-step ops on MI355X.

Argument marshalling only: every function takes torch tensors on a ROCm
device, passes their device pointers and the current HIP stream to the C ABI
of ``include/repro.h`` and returns.  All arithmetic runs in the library's
HIP kernels; there is no fallback, and a missing library is an error.

Entry points (same names as the C ABI):
    repro_gemm(A, B, trans_a=False, trans_b=False, out=None)
    repro_gemm_fma(A, B, trans_a=False, trans_b=False, out=None, variant=0)
    repro_tree_reduce(replicas, out=None, average=True)
    repro_replay_reduce(grads, dp_replicate, dp_shard, accum, out=None)
    repro_fold_push(slots, pushed, part);  repro_fold_result(slots, pushed, out, divisor=0)
    repro_adamw(state, grad, lr, beta1, beta2, eps, weight_decay, step)
    repro_state_hash(words, workspace=None) -> 32-byte digest (bytes)
    repro_state_hash_async(words, digest_out, workspace)
    repro_fp32_ops(op, a, b, out=None);  repro_fp32_fma(a, b, c, unit=0, out=None)
    repro_adamw_hash(state, grad, digest_out, workspace, lr, beta1, beta2, eps, weight_decay, step, chunk=0)
    repro_adamw_hash_noalloc(state, grad, digest_out, lr, beta1, beta2, eps, weight_decay, step)
    repro_grad_norm(grad, workspace=None, out=None) -> device tensor [norm, S]
    repro_adamw_bf16_step(w, m, v, grad, state, lr, beta1, beta2, eps, weight_decay,
                          max_norm=1.0, spike_threshold=5.0, skip_steps=5, workspace=None)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librepro.so")
_lib = None

REPRO_MAX_REPLICAS = 64
REPRO_MAX_REPLAY_BUFFERS = 384
REPRO_FOLD_SLOTS = 7


class ReproError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})")


def library():
    """Load librepro.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               f"g.build()'` (hipcc for gfx950); there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
        lib.repro_spec_version.restype = ctypes.c_char_p
        lib.repro_spec_version.argtypes = []
        lib.repro_strerror.restype = ctypes.c_char_p
        lib.repro_strerror.argtypes = [ctypes.c_int]
        gemm_args = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, i64, vp, i64, vp, i64]
        lib.repro_gemm.argtypes = gemm_args + [vp]
        lib.repro_gemm_variant.argtypes = gemm_args + [i32, vp]
        lib.repro_tree_reduce.argtypes = [vp, i32, i64, vp, i32, vp]
        lib.repro_tree_reduce_variant.argtypes = [vp, i32, i64, vp, i32, i32, vp]
        adamw_args = [vp, vp, i64, f32, f32, f32, f32, f32, i64]
        lib.repro_adamw.argtypes = adamw_args + [vp]
        lib.repro_adamw_variant.argtypes = adamw_args + [i32, vp]
        lib.repro_state_hash_workspace_bytes.restype = i64
        lib.repro_state_hash_workspace_bytes.argtypes = [i64]
        lib.repro_state_hash.argtypes = [vp, i64, vp, i64, vp, vp]
        lib.repro_fp32_ops.argtypes = [i32, vp, vp, vp, i64, vp]
        lib.repro_replay_reduce.argtypes = [vp, i32, i32, i32, i64, vp, vp]
        lib.repro_fold_push.argtypes = [vp, i32, vp, i64, vp]
        lib.repro_fold_result.argtypes = [vp, i32, i64, vp, i32, vp]
        lib.repro_gemm_fma.argtypes = gemm_args + [i32, vp]
        lib.repro_adamw_hash.argtypes = [vp, vp, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_float, i64, vp, i64, vp, i64, vp]
        lib.repro_grad_norm_workspace_bytes.restype = i64
        lib.repro_grad_norm_workspace_bytes.argtypes = [i64]
        lib.repro_grad_norm.argtypes = [vp, i32, i64, vp, i64, vp, vp]
        f32 = ctypes.c_float
        lib.repro_adamw_bf16_step.argtypes = [vp, vp, vp, vp, i32, i64, f32, f32, f32, f32, f32, f32, f32, i32, vp,
                                              i64, vp, vp]
        lib.repro_fp32_fma.argtypes = [vp, vp, vp, vp, i64, i32, vp]
        lib.repro_adamw_hash_noalloc.argtypes = [vp, vp, i64, f32, f32, f32, f32, f32, i64, vp, vp]
        for name in ("repro_gemm", "repro_gemm_variant", "repro_tree_reduce", "repro_tree_reduce_variant",
                     "repro_adamw", "repro_adamw_variant", "repro_state_hash", "repro_fp32_ops",
                     "repro_replay_reduce", "repro_fold_push", "repro_fold_result", "repro_gemm_fma",
                     "repro_fp32_fma", "repro_grad_norm", "repro_adamw_bf16_step", "repro_adamw_hash",
                     "repro_adamw_hash_noalloc"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return library().repro_strerror(int(status)).decode()


def spec_version() -> str:
    return library().repro_spec_version().decode()


def _check(status: int, what: str):
    if status != 0:
        raise ReproError(status, what)


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _on_device(t, name: str, dtype=None, min_bytes: int = 0):
    """Check that t is a contiguous tensor on the current ROCm device (of dtype, holding at least
    min_bytes): the library receives only its address, so a host or foreign-device tensor must
    never reach it."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on a ROCm device")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} must hold at least {min_bytes} bytes")
    return t


def _f32_device(t, name: str):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_cuda:
        raise TypeError(f"{name} must be a float32 tensor on a ROCm device")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return t


def _row_major(t, name: str):
    """(pointer, rows, cols, ld) of a 2-D float32 device tensor with unit column stride.

    The library reads row i at pointer + i * ld, so rows must not overlap: a view
    whose row stride is below its width (an expand() or an overlapping as_strided)
    is refused rather than passed with a larger ld that would address memory
    outside the tensor's storage."""
    _f32_device(t, name)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} needs unit stride along its last dimension")
    if rows > 1 and t.stride(0) < cols:
        raise ValueError(f"{name} has row stride {t.stride(0)} below its {cols} columns (overlapping rows)")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return t.data_ptr(), rows, cols, max(ld, 1)


def repro_gemm(A, B, trans_a: bool = False, trans_b: bool = False, out=None, variant: int = 0, stream=None,
               fused: bool = False):
    """C = op(A) @ op(B), one ascending-k unfused chain per output (fused: the
    declared fused multiply-add chain of repro_gemm_fma)."""
    import torch
    pa, ra, ca, lda = _row_major(A, "A")
    pb, rb, cb, ldb = _row_major(B, "B")
    M, K = (ca, ra) if trans_a else (ra, ca)
    K2, N = (cb, rb) if trans_b else (rb, cb)
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
    pc, rc, cc, ldc = _row_major(out, "out")
    if (rc, cc) != (M, N):
        raise ValueError("out has the wrong shape")
    lib = library()
    if fused:
        st = lib.repro_gemm_fma(int(trans_a), int(trans_b), M, N, K, pa, lda, pb, ldb, pc, ldc, int(variant),
                                _stream(stream))
    elif variant == 0:
        st = lib.repro_gemm(int(trans_a), int(trans_b), M, N, K, pa, lda, pb, ldb, pc, ldc, _stream(stream))
    else:
        st = lib.repro_gemm_variant(int(trans_a), int(trans_b), M, N, K, pa, lda, pb, ldb, pc, ldc, int(variant),
                                    _stream(stream))
    _check(st, "repro_gemm_fma" if fused else "repro_gemm")
    return out


def repro_gemm_fma(A, B, trans_a: bool = False, trans_b: bool = False, out=None, variant: int = 0, stream=None):
    """C = op(A) @ op(B) under the fused convention (0: matrix cores, 1: VALU)."""
    return repro_gemm(A, B, trans_a, trans_b, out, variant, stream, fused=True)


def repro_tree_reduce(replicas, out=None, average: bool = True, variant: int = 0, stream=None):
    """out = TreeFold(replicas) (times fl(1/R) when average)."""
    import torch
    reps = list(replicas)
    R = len(reps)
    if R < 1 or R > REPRO_MAX_REPLICAS:
        raise ValueError(f"need 1..{REPRO_MAX_REPLICAS} replicas")
    n = reps[0].numel()
    for i, r in enumerate(reps):
        _f32_device(r, f"replicas[{i}]")
        if r.numel() != n or not r.is_contiguous():
            raise ValueError("replicas must be contiguous and of equal size")
    if out is None:
        out = torch.empty_like(reps[0])
    _f32_device(out, "out")
    if out.numel() != n or not out.is_contiguous():
        raise ValueError("out must be contiguous with the replicas' size")
    ptrs = (ctypes.c_void_p * R)(*[r.data_ptr() for r in reps])
    lib = library()
    if variant == 0:
        st = lib.repro_tree_reduce(ctypes.cast(ptrs, ctypes.c_void_p), R, n, out.data_ptr(), int(bool(average)),
                                   _stream(stream))
    else:
        st = lib.repro_tree_reduce_variant(ctypes.cast(ptrs, ctypes.c_void_p), R, n, out.data_ptr(),
                                           int(bool(average)), int(variant), _stream(stream))
    _check(st, "repro_tree_reduce")
    return out


def _contiguous_f32(ts, name):
    n = ts[0].numel()
    for i, t in enumerate(ts):
        _f32_device(t, f"{name}[{i}]")
        if t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous and of equal size")
    return n


def repro_replay_reduce(grads, dp_replicate: int, dp_shard: int, accum: int, out=None, stream=None):
    """Algorithm 1's reduction of dp_replicate * dp_shard * accum microbatch gradients (mesh order)."""
    import torch
    gs = list(grads)
    if len(gs) != dp_replicate * dp_shard * accum or not gs:
        raise ValueError("need dp_replicate * dp_shard * accum gradient buffers")
    n = _contiguous_f32(gs, "grads")
    if out is None:
        out = torch.empty_like(gs[0])
    _contiguous_f32([gs[0], out], "out")
    ptrs = (ctypes.c_void_p * len(gs))(*[g.data_ptr() for g in gs])
    _check(library().repro_replay_reduce(ctypes.cast(ptrs, ctypes.c_void_p), dp_replicate, dp_shard, accum, n,
                                         out.data_ptr(), _stream(stream)), "repro_replay_reduce")
    return out


def _slot_ptrs(slots, n: int):
    import torch
    slots = list(slots)
    if len(slots) > REPRO_FOLD_SLOTS:
        raise ValueError(f"at most {REPRO_FOLD_SLOTS} slots")
    for i, t in enumerate(slots):
        if t is not None:
            _on_device(t, f"slots[{i}]", torch.float32)
            if t.numel() != n:
                raise ValueError(f"slots[{i}] must hold {n} floats")
    ptrs = [t.data_ptr() if t is not None else None for t in slots]
    ptrs += [None] * (REPRO_FOLD_SLOTS - len(ptrs))
    return (ctypes.c_void_p * REPRO_FOLD_SLOTS)(*ptrs)


def repro_fold_push(slots, pushed: int, part, stream=None):
    """Push one partial into the caller-owned level slots (list of device tensors or None)."""
    import torch
    _on_device(part, "part", torch.float32)
    ptrs = _slot_ptrs(slots, part.numel())
    _check(library().repro_fold_push(ctypes.cast(ptrs, ctypes.c_void_p), int(pushed), part.data_ptr(),
                                     part.numel(), _stream(stream)), "repro_fold_push")


def repro_fold_result(slots, pushed: int, out, divisor: int = 0, stream=None):
    import torch
    _on_device(out, "out", torch.float32)
    ptrs = _slot_ptrs(slots, out.numel())
    _check(library().repro_fold_result(ctypes.cast(ptrs, ctypes.c_void_p), int(pushed), out.numel(),
                                       out.data_ptr(), int(divisor), _stream(stream)), "repro_fold_result")
    return out


def repro_adamw(state, grad, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, step: int,
                variant: int = 0, stream=None):
    """In-place AdamW step on the flat state [w | m | v] (3n floats)."""
    _f32_device(state, "state")
    _f32_device(grad, "grad")
    n = grad.numel()
    if state.numel() != 3 * n or not state.is_contiguous() or not grad.is_contiguous():
        raise ValueError("state must be a contiguous [w | m | v] of 3 * grad.numel() floats")
    lib = library()
    args = (state.data_ptr(), grad.data_ptr(), n, float(lr), float(beta1), float(beta2), float(eps),
            float(weight_decay), int(step))
    if variant == 0:
        st = lib.repro_adamw(*args, _stream(stream))
    else:
        st = lib.repro_adamw_variant(*args, int(variant), _stream(stream))
    _check(st, "repro_adamw")
    return state


def repro_state_hash_workspace_bytes(n_words: int) -> int:
    v = library().repro_state_hash_workspace_bytes(int(n_words))
    if v < 0:
        raise ReproError(int(v), "repro_state_hash_workspace_bytes")
    return int(v)


def hash_workspace(n_words: int, device="cuda"):
    import torch
    return torch.empty(repro_state_hash_workspace_bytes(n_words), dtype=torch.uint8, device=device)


def repro_state_hash_async(words, digest_out, workspace, stream=None):
    """Enqueue the state hash; the 32-byte digest lands in ``digest_out`` (device uint8[32])."""
    import torch
    _on_device(words, "words", torch.float32)
    _on_device(digest_out, "digest_out", torch.uint8, 32)
    _on_device(workspace, "workspace", torch.uint8)
    st = library().repro_state_hash(words.data_ptr(), words.numel(), workspace.data_ptr(), workspace.numel(),
                                    digest_out.data_ptr(), _stream(stream))
    _check(st, "repro_state_hash")
    return digest_out


def repro_state_hash(words, workspace=None, stream=None) -> bytes:
    """32-byte state hash of the words (synchronises with the stream to return it)."""
    import torch
    if workspace is None:
        workspace = hash_workspace(words.numel(), words.device)
    digest = torch.empty(32, dtype=torch.uint8, device=words.device)
    repro_state_hash_async(words, digest, workspace, stream)
    return bytes(digest.cpu().numpy().tobytes())


def repro_adamw_hash(state, grad, digest_out, workspace, lr: float, beta1: float, beta2: float, eps: float,
                     weight_decay: float, step: int, chunk: int = 0, stream=None):
    """repro_adamw then the state hash of the updated state, fused into one pass (see repro.h)."""
    import torch
    _on_device(state, "state", torch.float32)
    _on_device(grad, "grad", torch.float32)
    _on_device(digest_out, "digest_out", torch.uint8, 32)
    _on_device(workspace, "workspace", torch.uint8)
    n = grad.numel()
    if state.numel() != 3 * n:
        raise ValueError("state must hold 3n floats for a grad of n")
    _check(library().repro_adamw_hash(state.data_ptr(), grad.data_ptr(), n, lr, beta1, beta2, eps, weight_decay,
                                      int(step), workspace.data_ptr(), workspace.numel(), digest_out.data_ptr(),
                                      int(chunk), _stream(stream)), "repro_adamw_hash")


REPRO_NOALLOC_SCRATCH_BYTES = 128 << 20


def repro_adamw_hash_noalloc(state, grad, digest_out, lr: float, beta1: float, beta2: float, eps: float,
                             weight_decay: float, step: int, stream=None):
    """repro_adamw_hash without a workspace: the library's per-device array holds the digests
    (calls overlapping on one device race; see repro.h)."""
    import torch
    _on_device(state, "state", torch.float32)
    _on_device(grad, "grad", torch.float32)
    _on_device(digest_out, "digest_out", torch.uint8, 32)
    n = grad.numel()
    if state.numel() != 3 * n:
        raise ValueError("state must hold 3n floats for a grad of n")
    _check(library().repro_adamw_hash_noalloc(state.data_ptr(), grad.data_ptr(), n, lr, beta1, beta2, eps,
                                              weight_decay, int(step), digest_out.data_ptr(), _stream(stream)),
           "repro_adamw_hash_noalloc")


def repro_fp32_ops(op: int, a, b=None, out=None, stream=None):
    """One contract operation per element (diagnostic; see repro.h)."""
    import torch
    _f32_device(a, "a")
    b = a if b is None else b
    _f32_device(b, "b")
    if out is None:
        out = torch.empty_like(a)
    if not (a.is_contiguous() and b.is_contiguous() and out.is_contiguous()) or a.numel() != b.numel():
        raise ValueError("a, b, out must be contiguous and of equal size")
    _check(library().repro_fp32_ops(int(op), a.data_ptr(), b.data_ptr(), out.data_ptr(), a.numel(),
                                    _stream(stream)), "repro_fp32_ops")
    return out


def repro_fp32_fma(a, b, c, unit: int = 0, out=None, stream=None):
    """out = fma(a, b, c) per element on one unit (0: v_fma_f32; 1, 2, 3: the matrix-core
    instructions 32x32x1_2b, 16x16x1_4b, 4x4x1_16b)."""
    import torch
    for t, nm in ((a, "a"), (b, "b"), (c, "c")):
        _f32_device(t, nm)
    if out is None:
        out = torch.empty_like(a)
    ts = (a, b, c, out)
    if not all(t.is_contiguous() for t in ts) or len({t.numel() for t in ts}) != 1:
        raise ValueError("a, b, c, out must be contiguous and of equal size")
    _check(library().repro_fp32_fma(a.data_ptr(), b.data_ptr(), c.data_ptr(), out.data_ptr(), a.numel(), int(unit),
                                    _stream(stream)), "repro_fp32_fma")
    return out


REPRO_GRAD_F32, REPRO_GRAD_BF16 = 0, 1
STEP_STATE_BYTES = 32
# Field layout of repro_step_state (include/repro.h).
STEP_STATE_FIELDS = [("step", "<i8"), ("skip_left", "<i4"), ("applied", "<i4"), ("beta1_pow", "<f4"),
                     ("beta2_pow", "<f4"), ("grad_norm", "<f4"), ("clip_coef", "<f4")]


def _grad_dtype(g):
    import torch
    if g.dtype == torch.bfloat16:
        return REPRO_GRAD_BF16
    if g.dtype == torch.float32:
        return REPRO_GRAD_F32
    raise TypeError("grad must be float32 or bfloat16")


def grad_norm_workspace(n: int, device="cuda"):
    import torch
    nbytes = int(library().repro_grad_norm_workspace_bytes(int(n)))
    if nbytes < 0:
        raise ValueError("bad size")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def new_step_state(device="cuda"):
    """A zeroed repro_step_state in device memory (no step taken yet)."""
    import torch
    return torch.zeros(STEP_STATE_BYTES, dtype=torch.uint8, device=device)


def read_step_state(state) -> dict:
    """Host copy of a device repro_step_state as a dict."""
    import numpy as np
    rec = state.cpu().numpy().view(np.dtype(STEP_STATE_FIELDS))[0]
    return {name: rec[name].item() for name, _ in STEP_STATE_FIELDS}


def repro_grad_norm(grad, workspace=None, out=None, stream=None):
    """Device tensor [norm, S]: the pre-clip global norm of a flat float32 or bfloat16 gradient."""
    import torch
    _on_device(grad, "grad")
    if workspace is None:
        workspace = grad_norm_workspace(grad.numel(), grad.device)
    if out is None:
        out = torch.empty(2, dtype=torch.float32, device=grad.device)
    _on_device(workspace, "workspace", torch.uint8)
    _on_device(out, "out", torch.float32, 8)
    _check(library().repro_grad_norm(grad.data_ptr(), _grad_dtype(grad), grad.numel(), workspace.data_ptr(),
                                     workspace.numel(), out.data_ptr(), _stream(stream)), "repro_grad_norm")
    return out


def repro_adamw_bf16_step(w, m, v, grad, state, lr: float, beta1: float, beta2: float, eps: float,
                          weight_decay: float, max_norm: float = 1.0, spike_threshold: float = 5.0,
                          skip_steps: int = 5, workspace=None, stream=None):
    """One BF16-parameter optimizer step in place (w bfloat16; m, v float32; grad float32 or bfloat16)."""
    import torch
    if w.dtype != torch.bfloat16 or m.dtype != torch.float32 or v.dtype != torch.float32:
        raise TypeError("w must be bfloat16, m and v float32")
    n = w.numel()
    for t, nm in ((w, "w"), (m, "m"), (v, "v"), (grad, "grad")):
        _on_device(t, nm)
        if t.numel() != n:
            raise ValueError(f"{nm} must hold {n} elements")
    _on_device(state, "state", torch.uint8, STEP_STATE_BYTES)
    if workspace is None:
        workspace = grad_norm_workspace(n, w.device)
    _on_device(workspace, "workspace", torch.uint8)
    _check(library().repro_adamw_bf16_step(w.data_ptr(), m.data_ptr(), v.data_ptr(), grad.data_ptr(),
                                           _grad_dtype(grad), n, lr, beta1, beta2, eps, weight_decay, max_norm,
                                           spike_threshold, int(skip_steps), workspace.data_ptr(), workspace.numel(),
                                           state.data_ptr(), _stream(stream)), "repro_adamw_bf16_step")


__all__ = ["repro_gemm", "repro_adamw_hash", "repro_adamw_hash_noalloc", "REPRO_NOALLOC_SCRATCH_BYTES", "repro_grad_norm", "repro_adamw_bf16_step", "new_step_state", "read_step_state",
           "grad_norm_workspace", "repro_gemm_fma", "repro_fp32_fma", "repro_tree_reduce", "repro_replay_reduce", "repro_fold_push", "repro_fold_result", "repro_adamw", "repro_state_hash", "repro_state_hash_async",
           "repro_state_hash_workspace_bytes", "repro_fp32_ops", "hash_workspace", "spec_version", "library",
           "ReproError", "LIB_PATH"]
