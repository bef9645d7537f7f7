"""The flat optimizer checkpoint record used by the resume tests.

Layout (the checkpoint page's file format): a little-endian int32 step, a
little-endian int32 parameter count n, then the 12n bytes of [w | m | v] as
little-endian binary32 words.  Saving the moments with the weights is what
makes a resumed run bit-identical to one that never stopped (the same page).
The step stored is the last step applied; the next update uses step + 1.
This is test harness code: the library itself does no I/O.
"""
import os
import struct

import numpy as np


def write_record(path: str, step: int, state) -> None:
    state = np.ascontiguousarray(state, dtype="<f4").reshape(-1)
    n = state.size // 3
    assert state.size == 3 * n and 0 <= n < 2**31 and 0 <= step < 2**31
    tmp = path + ".tmp"
    with open(tmp, "wb") as fh:
        fh.write(struct.pack("<ii", step, n))
        fh.write(state.tobytes())
        fh.flush()
        os.fsync(fh.fileno())
    os.replace(tmp, path)  # a reader never sees a half-written record


def read_record(path: str):
    with open(path, "rb") as fh:
        head = fh.read(8)
        step, n = struct.unpack("<ii", head)
        body = fh.read()
    if len(body) != 12 * n:
        raise ValueError(f"record holds {len(body)} bytes of state, expected {12 * n}")
    return step, np.frombuffer(body, dtype="<f4").astype(np.float32)
