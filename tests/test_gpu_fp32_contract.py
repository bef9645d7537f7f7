"""GPU: the binary32 contract at its edges (flush boundary, division, sqrt).

OPEN-1B paper, section 2.1 ("Fused multiply-add", "Subnormals") and Table 1.
repro_fp32_ops runs one operation per element with the device arithmetic of
the kernels (every kernel runs in the same hardware flush mode, so its
v_mul_f32 and v_add_f32 are also the GEMM's).  Every result is compared with
the oracle's contract operation: the x86 FTZ/DAZ operation of the host.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_amd as br
import oracle
from parity_util import assert_bitwise, to_dev, to_host

pytestmark = pytest.mark.gpu

# GPU op -> oracle op
OPS = {0: oracle.OP_ADD, 1: oracle.OP_SUB, 2: oracle.OP_MUL, 3: oracle.OP_DIV, 4: oracle.OP_SQRT}


def _bits(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def _boundary_operands():
    """Operand pairs whose exact results sit at or near 2^-126."""
    a, b = [], []
    # Products m * 2^-126 and m * 2^-127 for mantissas m just below 1 and 2:
    # exact results around the smallest normal, including the tie
    # (1 - 2^-24) * 2^-126 = 2^-126 - 2^-150.
    for mant in range(0x3F7FFF00, 0x3F800100):
        for e in (2.0 ** -126, 2.0 ** -127, -(2.0 ** -126)):
            a.append(_bits(mant))
            b.append(np.float32(e))
    for mant in range(0x3FFFFF00, 0x40000000):
        a.append(_bits(mant))
        b.append(np.float32(2.0 ** -127))
    # Pairs of moderate numbers whose product lands near 2^-126: x * y with
    # x = 2^-63 * (1 + i 2^-23), y = 2^-63 * (1 - j 2^-24).
    for i in range(0, 64):
        for j in range(0, 64):
            a.append(np.float32(2.0 ** -63 * (1 + i * 2.0 ** -23)))
            b.append(np.float32(2.0 ** -63 * (1 - j * 2.0 ** -24)))
    # Subnormal operands, signed zeros, the smallest normal.
    specials = [0.0, -0.0, 2.0 ** -149, -(2.0 ** -149), 2.0 ** -127, 2.0 ** -126, -(2.0 ** -126), 1.0, -1.5,
                2.0 ** 127, 3.0]
    for x in specials:
        for y in specials:
            a.append(np.float32(x))
            b.append(np.float32(y))
    return np.array(a, np.float32), np.array(b, np.float32)


def _division_operands():
    """Quotients whose exact value sits at or near 2^-126."""
    a, b = [], []
    divisors = [2.0, 1.0, 3.0, 1.5, 0.75]
    divisors += [float(_bits(u)) for u in (0x40000001, 0x3FFFFFFF, 0x3F800001, 0x3F7FFFFF, 0x3FC00001)]
    for u in list(range(0x00FFFF00, 0x01000100)) + list(range(0x00800000, 0x00800100)) + \
            list(range(0x00BFFF00, 0x00C00100)):
        for d in divisors:
            a.append(_bits(u))
            b.append(np.float32(d))
            a.append(-_bits(u))
            b.append(np.float32(d))
    return np.array(a, np.float32), np.array(b, np.float32)


@pytest.mark.parametrize("op", [0, 1, 2, 3])
def test_boundary_cases(op):
    a, b = _boundary_operands()
    if op == 3:
        a, b = _division_operands()
    ref = oracle.fp32_op(OPS[op], a, b)
    got = to_host(br.repro_fp32_ops(op, to_dev(a), to_dev(b)))
    finite = np.isfinite(ref)
    assert_bitwise(got[finite], ref[finite], f"op {op}")


@pytest.mark.parametrize("op", [0, 1, 2, 3])
def test_random_operands_wide_exponents(op):
    rng = np.random.default_rng(op)
    n = 4_000_000
    a = (rng.standard_normal(n) * np.exp2(rng.uniform(-70, 70, n))).astype(np.float32)
    b = (rng.standard_normal(n) * np.exp2(rng.uniform(-70, 70, n))).astype(np.float32)
    ref = oracle.fp32_op(OPS[op], a, b)
    got = to_host(br.repro_fp32_ops(op, to_dev(a), to_dev(b)))
    finite = np.isfinite(ref)
    assert_bitwise(got[finite], ref[finite], f"op {op}")


def test_sqrt_exhaustive_over_all_non_negative_floats():
    # Every binary32 bit pattern from +0 to +inf (2^31 inputs, in chunks).
    chunk = 1 << 27
    for start in range(0, 0x7F800001, chunk):
        stop = min(start + chunk, 0x7F800001)
        bits = torch.arange(start, stop, dtype=torch.int64, device="cuda").to(torch.int32)
        x = bits.view(torch.float32)
        got = to_host(br.repro_fp32_ops(4, x))
        ref = oracle.fp32_op(oracle.OP_SQRT, to_host(x))
        assert_bitwise(got, ref, f"sqrt chunk at 0x{start:08x}")


def _near_min_normal_products(n, seed):
    """Random pairs whose products fall within a few ulps of +-2^-126."""
    rng = np.random.default_rng(seed)
    a = np.ldexp(rng.uniform(1, 2, n), rng.integers(-80, -46, n)).astype(np.float32)
    b = (2.0 ** -126 / a.astype(np.float64)).astype(np.float32)
    b = (b.view(np.int32) + rng.integers(-3, 4, n).astype(np.int32)).view(np.float32)
    return (a * rng.choice([-1, 1], n).astype(np.float32)).astype(np.float32), b


def test_products_around_the_smallest_normal():
    # About 5% of these products are exactly the cases where "tiny after
    # rounding with an unbounded exponent" and "subnormal after rounding to
    # the subnormal grid" disagree; the GPU must follow the oracle's rule.
    a, b = _near_min_normal_products(2_000_000, 11)
    ref = oracle.fp32_op(oracle.OP_MUL, a, b)
    got = to_host(br.repro_fp32_ops(2, to_dev(a), to_dev(b)))
    assert_bitwise(got, ref, "products near 2^-126")
    assert (ref == 0).sum() > 10_000 and (np.abs(ref) == np.float32(2.0 ** -126)).sum() > 10_000


def test_unfused_multiply_then_add():
    # -1 + fl((1 + 2^-12)^2) = 2^-11 through the device multiply and add.
    t = torch.full((4,), 1.0 + 2.0 ** -12, device="cuda")
    p = br.repro_fp32_ops(2, t, t)
    s = br.repro_fp32_ops(0, torch.full((4,), -1.0, device="cuda"), p)
    assert (to_host(s) == np.float32(2.0 ** -11)).all()
