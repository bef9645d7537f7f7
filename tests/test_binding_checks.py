"""The Python binding refuses host tensors before any call into the library.

The C ABI receives bare addresses, so a host tensor passed through would hand
a host pointer to a GPU kernel.  These checks run on the CPU: every wrapper
must raise before it reaches a compute entry point.
"""
import pytest
import torch

import bitwise_reproducible_amd as br

F32 = torch.float32


def _host(n=1024, dtype=F32):
    return torch.zeros(n, dtype=dtype)


CASES = {
    "repro_gemm": lambda: br.repro_gemm(torch.zeros(4, 4), torch.zeros(4, 4)),
    "repro_gemm_fma": lambda: br.repro_gemm_fma(torch.zeros(4, 4), torch.zeros(4, 4)),
    "repro_tree_reduce": lambda: br.repro_tree_reduce([_host(), _host()]),
    "repro_replay_reduce": lambda: br.repro_replay_reduce([_host()] * 2, 1, 2, 1),
    "repro_fold_push": lambda: br.repro_fold_push([None] * br.REPRO_FOLD_SLOTS, 0, _host()),
    "repro_fold_result": lambda: br.repro_fold_result([_host()], 1, _host()),
    "repro_adamw": lambda: br.repro_adamw(_host(3 * 1024), _host(), 1e-3, 0.9, 0.999, 1e-8, 0.1, 1),
    "repro_state_hash_async": lambda: br.repro_state_hash_async(_host(), _host(32, torch.uint8),
                                                                _host(4096, torch.uint8)),
    "repro_adamw_hash": lambda: br.repro_adamw_hash(_host(3 * 1024), _host(), _host(32, torch.uint8),
                                                    _host(4096, torch.uint8), 1e-3, 0.9, 0.999, 1e-8, 0.1, 1),
    "repro_adamw_hash_noalloc": lambda: br.repro_adamw_hash_noalloc(_host(3 * 1024), _host(),
                                                                    _host(32, torch.uint8), 1e-3, 0.9, 0.999,
                                                                    1e-8, 0.1, 1),
    "repro_fp32_ops": lambda: br.repro_fp32_ops(0, _host(), _host()),
    "repro_fp32_fma": lambda: br.repro_fp32_fma(_host(), _host(), _host()),
    "repro_grad_norm": lambda: br.repro_grad_norm(_host(), workspace=_host(4096, torch.uint8),
                                                  out=_host(2)),
    "repro_adamw_bf16_step": lambda: br.repro_adamw_bf16_step(
        _host(dtype=torch.bfloat16), _host(), _host(), _host(), _host(32, torch.uint8), 1e-3, 0.9, 0.95, 1e-8,
        0.1, workspace=_host(4096, torch.uint8)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_host_tensor_is_refused(name):
    with pytest.raises(TypeError, match="ROCm device"):
        CASES[name]()


def test_every_compute_wrapper_is_covered():
    compute = {n for n in br.__all__ if n.startswith("repro_") and n != "repro_state_hash_workspace_bytes"}
    compute.discard("repro_state_hash")  # allocates its digest on the words' device, then calls the async form
    assert compute <= set(CASES), sorted(compute - set(CASES))


def test_overlapping_rows_are_refused(monkeypatch):
    # The GEMM reads row i at base + i * ld.  A view whose row stride is below
    # its width (expand, an overlapping as_strided) would make the library read
    # or write past the storage, so the binding refuses it before any call.  The
    # device check is bypassed so that host tensors can stand in (no call is made).
    monkeypatch.setattr(br, "_f32_device", lambda t, name: t)
    expanded = torch.zeros(1, 64).expand(64, 64)
    with pytest.raises(ValueError, match="overlapping rows"):
        br._row_major(expanded, "A")
    overlap = torch.zeros(200).as_strided((8, 64), (16, 1))
    with pytest.raises(ValueError, match="overlapping rows"):
        br._row_major(overlap, "out")
    with pytest.raises(ValueError, match="overlapping rows"):
        br.repro_gemm(torch.zeros(64, 64), expanded)
    with pytest.raises(ValueError, match="overlapping rows"):
        br.repro_gemm(torch.zeros(64, 64), torch.zeros(64, 64), out=torch.zeros(64).expand(64, 64))
    # Accepted views keep their own row stride as ld.
    base = torch.zeros(10, 80)
    assert br._row_major(base[:, 8:72], "A")[1:] == (10, 64, 80)
    assert br._row_major(torch.zeros(1, 5), "A")[1:] == (1, 5, 5)
    assert br._row_major(torch.zeros(7, 1)[:, :1], "A")[1:] == (7, 1, 1)
