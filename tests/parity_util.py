"""Helpers shared by the GPU parity tests (comparison and device transfer)."""
import numpy as np


def differing_words(a, b) -> np.ndarray:
    """Indices where two float32 arrays differ as 32-bit words."""
    a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1).view(np.uint32)
    b = np.ascontiguousarray(b, dtype=np.float32).reshape(-1).view(np.uint32)
    assert a.shape == b.shape, (a.shape, b.shape)
    return np.nonzero(a != b)[0]


def assert_bitwise(got, ref, what: str = "output"):
    """0 differing words, with a readable report of the first mismatches."""
    got = np.ascontiguousarray(got, dtype=np.float32).reshape(-1)
    ref = np.ascontiguousarray(ref, dtype=np.float32).reshape(-1)
    bad = differing_words(got, ref)
    if bad.size:
        rows = [f"  [{i}] got {got[i]!r} (0x{got.view(np.uint32)[i]:08x}) want {ref[i]!r} "
                f"(0x{ref.view(np.uint32)[i]:08x})" for i in bad[:8]]
        raise AssertionError(f"{what}: {bad.size} of {got.size} words differ\n" + "\n".join(rows))


def to_dev(x, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


def to_host(t) -> np.ndarray:
    return t.detach().cpu().numpy()
