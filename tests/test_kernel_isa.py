"""Instruction audit of the library's own kernels (CPU only: hipcc emits the
gfx950 assembly of our sources, nothing is run).

The binary32 contract keeps multiply and add unfused (OPEN-1B paper, section
2.1 "Fused multiply-add"): no kernel other than those of the declared fused
convention may contain a fused or packed fp32 instruction.  The fused-chain
kernels must contain them, and the matrix-core fused GEMM must do all of its
arithmetic on the matrix cores.  No kernel may spill to scratch memory.
"""
import re
import sys
from collections import Counter
from concurrent.futures import ThreadPoolExecutor

import pytest

sys.path.insert(0, __import__("os").path.join(__import__("os").path.dirname(__file__), "..",
                                               "bitwise_reproducible_amd", "csrc"))
import build as lib_build  # noqa: E402

SOURCES = ["gemm.hip", "elementwise.hip", "replay.hip", "state_hash.hip", "fused.hip", "optimizer.hip"]
FUSED_OR_PACKED = re.compile(r"^v_(fma|fmac|mac|mad)_f32|^v_pk_(fma|add|mul)_f32|^v_(fma|mad)_mix|^v_fma_legacy")
# Kernels of the declared fused convention.
FUSED_KERNELS = ("k_gemm_fma", "k_gemm_mfma_fma", "k_fma_valu", "k_fma_mfma")


def _kernels(asm: str):
    out = {}
    for part in re.split(r"\n(?=_Z[^\s:]+:)", asm):
        m = re.match(r"(_Z[^\s:]+):", part)
        if m:
            body = part.split(".Lfunc_end")[0]
            out[m.group(1)] = Counter(re.findall(r"^\s+(v_[a-z0-9_]+)", body, re.M))
    meta = {}
    for m in re.finditer(r"\.name:\s+(_Z\S+)\n(?:\s+\.[^\n]*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)", asm):
        meta[m.group(1)] = int(m.group(2))
    return out, meta


def _short(mangled: str) -> str:
    m = re.search(r"(k_[a-z0-9_]+)", mangled)
    return m.group(1) if m else mangled


@pytest.fixture(scope="module")
def asms():
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(lib_build.disassemble, SOURCES)))


@pytest.fixture(scope="module")
def kernels(asms):
    ks, meta = {}, {}
    for a in asms.values():
        k, m = _kernels(a)
        ks.update(k)
        meta.update(m)
    assert len(ks) >= 40, sorted(ks)
    return ks, meta


def test_only_fused_convention_kernels_fuse(kernels):
    # The compiler's correctly rounded division (v_div_scale, v_rcp, fma
    # refinement, v_div_fmas, v_div_fixup) and square root (v_rsq and fma
    # refinement) use fused steps internally; those sequences round once to
    # the IEEE result (checked exhaustively for sqrt and on boundary sets for
    # division by the GPU tests).  Each may bring at most 5 fused
    # instructions; every other fused or packed fp32 instruction is an error.
    ks, _ = kernels
    for name, ops in ks.items():
        if _short(name) in FUSED_KERNELS:
            continue
        packed = {op: c for op, c in ops.items() if op.startswith("v_pk_")}
        assert not packed, f"{_short(name)} ({name}) has packed fp32 instructions: {packed}"
        fused = sum(c for op, c in ops.items() if FUSED_OR_PACKED.match(op))
        allowed = 5 * (ops["v_div_fixup_f32"] + ops["v_rsq_f32_e32"])
        assert fused <= allowed, f"{_short(name)} ({name}): {fused} fused instructions, {allowed} allowed"
        if _short(name).startswith(("k_gemm", "k_tree_reduce", "k_replay", "k_fold", "k_hash", "k_norm_fold")):
            assert fused == 0, f"{_short(name)} has fused instructions"


def test_fused_kernels_use_the_declared_units(kernels):
    ks, _ = kernels
    seen = set()
    for name, ops in ks.items():
        s = _short(name)
        if s == "k_gemm_mfma_fma":
            assert ops["v_mfma_f32_32x32x1_2b_f32"] >= 32
            assert ops["v_add_f32_e32"] == 0 and ops["v_add_f32_e64"] == 0
            assert not any(FUSED_OR_PACKED.match(op) for op in ops)
        elif s == "k_gemm_fma":
            assert ops["v_fmac_f32_e32"] + ops["v_fma_f32"] >= 2048  # 32 k steps x 8 x 8 outputs per lane
            assert ops["v_add_f32_e32"] == 0
        elif s == "k_fma_mfma":
            # One K = 1 matrix instruction per instantiation (32x32, 16x16 or 4x4 blocks).
            shapes = [op for op in ("v_mfma_f32_32x32x1_2b_f32", "v_mfma_f32_16x16x1_4b_f32",
                                    "v_mfma_f32_4x4x1_16b_f32") if ops[op]]
            assert len(shapes) == 1 and ops[shapes[0]] == 1, ops
            assert not any(FUSED_OR_PACKED.match(op) for op in ops)
        elif s == "k_fma_valu":
            assert ops["v_fmac_f32_e32"] + ops["v_fma_f32"] >= 1
        else:
            continue
        seen.add(s)
    assert seen == set(FUSED_KERNELS)


def test_unfused_gemm_chain_is_one_multiply_and_one_add_per_step(kernels):
    ks, _ = kernels
    seen = 0
    for name, ops in ks.items():
        if _short(name) == "k_gemm" and "Li128ELi128ELi32ELi8ELi8E" in name:
            # 32 k steps x 8 x 8 outputs per lane in the unrolled slab loop.
            assert ops["v_mul_f32_e32"] >= 2048 and ops["v_add_f32_e32"] >= 2048, ops
            seen += 1
    assert seen == 8  # the default kernel, 4 transposes x 2 load widths
    seen = 0
    for name, ops in ks.items():
        if _short(name) == "k_gemm" and "Li256ELi128ELi16ELi16ELi8E" in name:
            # The large-output kernel: 16 k steps x 16 x 8 outputs per lane.
            assert ops["v_mul_f32_e32"] >= 2048 and ops["v_add_f32_e32"] >= 2048, ops
            seen += 1
    assert seen == 8


def _loops(body: str):
    """Instruction counts of each loop (a label and the branch back to it)."""
    lines = body.split("\n")
    out = []
    for i, line in enumerate(lines):
        m = re.match(r"(\.LBB\d+_\d+):", line)
        if not m:
            continue
        for j in range(i + 1, len(lines)):
            if re.search(r"s_(cbranch_\w+|branch) " + re.escape(m.group(1)) + r"$", lines[j]):
                out.append(Counter(re.findall(r"^\s+([a-z_0-9]+)", "\n".join(lines[i:j]), re.M)))
                break
    return out


def test_interior_slab_loop_is_branch_free(asms):
    # The GEMMs with 16-byte loads run interior tiles through a slab loop with
    # unchecked loads from a uniform base: no exec-mask branches, no register
    # copies (a join of two compute paths in the loop once copied every
    # accumulator on each pass), one 64-bit address add per load.
    asm = asms["gemm.hip"]
    seen = Counter()
    for part in re.split(r"\n(?=_Z[^\s:]+:)", asm):
        m = re.match(r"(_Z[^\s:]+):", part)
        if not m:
            continue
        name = m.group(1)
        if re.search(r"k_gemm(_fma)?ILi(256|128)ELi128E.*ELb1EEEv", name):
            # VALU tiles: BK steps x TM x TN multiplies (or fused steps).
            def is_slab(c):
                return c["v_mul_f32_e32"] + c["v_fmac_f32_e32"] + c["v_fma_f32"] >= 2048
        elif re.search(r"k_gemm_mfma(_fma)?ILi32ELb[01]ELb[01]ELb1EEEv", name):
            # Matrix-core tiles, 32-deep slabs: two 32x32 products per k step;
            # the unfused kernel adds each product on the VALU (2 x 32 adds
            # per step).
            fused = "k_gemm_mfma_fma" in name
            bk = 32

            def is_slab(c, bk=bk, fused=fused):
                return (c["v_mfma_f32_32x32x1_2b_f32"] == 2 * bk
                        and c["v_add_f32_e32"] == (0 if fused else 64 * bk) and c["global_load_dwordx4"] >= 1)
        else:
            continue
        loops = _loops(part.split(".Lfunc_end")[0])
        interior = [c for c in loops if is_slab(c) and c["s_and_saveexec_b64"] == 0]
        assert len(interior) == 1, (_short(name), name)
        c = interior[0]
        assert c["v_mov_b32_e32"] == 0, (name, c["v_mov_b32_e32"])
        assert 1 <= c["global_load_dwordx4"] <= 8 and c["v_lshl_add_u64"] <= c["global_load_dwordx4"] + 2, (
            name, c)
        seen[_short(name)] += 1
    # Two VALU tile shapes and one matrix-core shape, 4 transposes each.
    assert seen == {"k_gemm": 8, "k_gemm_fma": 8, "k_gemm_mfma": 4, "k_gemm_mfma_fma": 4}, seen


def test_no_kernel_uses_scratch(kernels):
    ks, meta = kernels
    assert set(meta) >= set(ks)
    spilled = {_short(k): v for k, v in meta.items() if v}
    assert not spilled, spilled


def test_hash_compression_instruction_mix(kernels):
    # The hash rows' bounds count ~2,000 VALU instructions per 128-byte block,
    # 1,153 of them half-rate opcodes: per G function 6 v_lshl_add_u64 (64-bit
    # adds), 6 v_alignbit_b32 (rotations by 24, 16, 63; by 32 is a swap) and 8
    # v_xor_b32; 96 G per block.  Each kernel below holds one compression body
    # (k_hash_leaves<true> two: whole leaves and the word-by-word tail).
    ks, _ = kernels
    bodies = {"k_adamw_hash_leaves": 1, "k_hash_level": 1, "k_hash_tail": 1}
    seen = set()
    for name, ops in ks.items():
        s = _short(name)
        k = bodies.get(s, 2 if "hash_leavesILb1" in name else 1 if s == "k_hash_leaves" else 0)
        if not k:
            continue
        assert ops["v_alignbit_b32"] == 576 * k, (s, ops["v_alignbit_b32"])
        assert 576 * k <= ops["v_lshl_add_u64"] <= 576 * k + 16, (s, ops["v_lshl_add_u64"])
        assert 784 * k <= ops["v_xor_b32_e32"] <= (784 + 30) * k, (s, ops["v_xor_b32_e32"])
        seen.add(name)
    assert len(seen) == 5
