"""GPU check of repro_adamw_hash_noalloc against repro_adamw_hash.

The no-allocation entry point keeps the hash digests in the library's own
per-device array instead of a caller workspace.  Its results must equal the
workspace form bit for bit (the updated [w | m | v] and the 32-byte state
hash), call after call: the second call here is smaller than the first, so
digests left in the array by the first call must not leak into the second.
Also the in-turn path (n not a multiple of 1024) and the size limit.
"""
import ctypes

import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
import synth
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)


def _inputs(n, tag):
    st = np.concatenate([synth.generate(n, synth.NORMAL, synth.tid(0x0A, tag), 0.02),
                         synth.generate(n, synth.NORMAL, synth.tid(0x0A, tag + 1), 1e-4),
                         synth.generate(n, synth.HALF_NORMAL, synth.tid(0x0A, tag + 2), 1e-6)])
    return st, synth.generate(n, synth.NORMAL, synth.tid(0x0A, tag + 3), 1e-3)


def _both(n, tag, step):
    """(state, digest) from the no-allocation call and from repro_adamw_hash."""
    st, g = _inputs(n, tag)
    dg = to_dev(g)
    a, b = to_dev(st), to_dev(st)
    da = torch.empty(32, dtype=torch.uint8, device="cuda")
    db = torch.empty(32, dtype=torch.uint8, device="cuda")
    br.repro_adamw_hash_noalloc(a, dg, da, step=step, **HP)
    br.repro_adamw_hash(b, dg, db, br.hash_workspace(3 * n), step=step, **HP)
    torch.cuda.synchronize()
    return (to_host(a), bytes(to_host(da))), (to_host(b), bytes(to_host(db))), (st, g)


def test_two_calls_in_a_row_match_the_workspace_form():
    # Fused path (n a multiple of 1024): a larger call, then a smaller one.
    for n, tag, step in ((1024 * 1500, 0x10, 1000), (1024 * 37, 0x20, 3)):
        print(f"no-alloc fused n={n} step={step}", flush=True)
        (sa, da), (sb, db), (st, g) = _both(n, tag, step)
        assert_bitwise(sa, sb, f"state n={n}")
        assert da == db, f"digest n={n}"
        if n <= 1024 * 37:  # and both are the oracle's
            oracle.adamw_inplace(st, g, step=step, **HP)
            assert_bitwise(sa, st, f"oracle state n={n}")
            assert da == oracle.state_hash(st)


def test_in_turn_path_and_repeat():
    # n not a multiple of 1024: the update and the hash run in turn; then the
    # same call again gives the same digest.
    for n, tag in ((5003, 0x30), (1, 0x40), (100_000, 0x50)):
        print(f"no-alloc in-turn n={n}", flush=True)
        (sa, da), (sb, db), _ = _both(n, tag, 7)
        assert_bitwise(sa, sb, f"state n={n}")
        assert da == db, f"digest n={n}"
    (sa2, da2), _, _ = _both(100_000, 0x50, 7)
    assert da2 == da and np.array_equal(sa2.view(np.uint32), sa.view(np.uint32))


def test_limit_and_errors():
    lib = br.library()
    d = torch.zeros(4096, device="cuda")
    dig = torch.zeros(32, dtype=torch.uint8, device="cuda")
    p, q = d.data_ptr(), dig.data_ptr()
    # The largest n whose hash fits the array, and the first that does not.
    limit = br.REPRO_NOALLOC_SCRATCH_BYTES
    assert br.repro_state_hash_workspace_bytes(3 * 1_200_000_000) <= limit
    assert br.repro_state_hash_workspace_bytes(3 * 1_400_000_000) > limit
    args = (1e-3, 0.9, 0.999, 1e-8, 0.1)
    # Rejected on the host, before anything is enqueued.
    assert lib.repro_adamw_hash_noalloc(p, p, 1_400_000_000, *args, 1, q, None) == -4
    assert lib.repro_adamw_hash_noalloc(p, p, 2**62, *args, 1, q, None) == -4
    assert lib.repro_adamw_hash_noalloc(p, p, 16, *args, 0, q, None) == -1
    assert lib.repro_adamw_hash_noalloc(p, p, 16, *args, 1, None, None) == -1
    assert lib.repro_adamw_hash_noalloc(p, p, 16, *args, 1, q + 4, None) == -2
    assert lib.repro_adamw_hash_noalloc(p, p + 2, 16, *args, 1, q, None) == -2
    # n = 0: the hash of an empty state (one empty leaf and its root).
    assert lib.repro_adamw_hash_noalloc(None, None, 0, *args, 1, q, None) == 0
    torch.cuda.synchronize()
    assert bytes(to_host(dig)) == oracle.state_hash(np.zeros(0, np.float32))
