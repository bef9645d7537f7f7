"""The oracle's pins are not vacuous: each plausible mistake, planted in a copy
of the oracle source and compiled on the CPU, makes at least one pin fail.

Nothing here touches the GPU library or the committed oracle build.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle import build as oracle_build

import test_oracle_adamw as T_ADAMW
import test_oracle_adamw_bf16 as T_BF16
import test_oracle_fma as T_FMA
import test_oracle_fp32 as T_FP32
import test_oracle_gemm as T_GEMM
import test_oracle_hash as T_HASH
import test_oracle_replay as T_REPLAY
import test_oracle_tree_reduce as T_TREE

SRC = oracle_build.SRC

# (name, text to find, replacement, pins that must fail)
MUTATIONS = [
    ("gemm_descending_k", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = K - 1; k >= 0; --k)",
     [T_GEMM.test_ascending_k_order_witness]),
    ("gemm_fused_mac", "acc = f_add(acc, f_mul(a, b));", "acc = fmaf(a, b, acc);",
     [T_GEMM.test_unfused_multiply_add_witness]),
    ("gemm_transposed_a", "float a = trans_a ? A[k * lda + i] : A[i * lda + k];",
     "float a = trans_a ? A[i * lda + k] : A[k * lda + i];",
     [lambda: T_GEMM.test_exact_integer_products(0, 0, 3, 5, 7)]),
    ("gemm_dropped_last_term", "for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)",
     [lambda: T_GEMM.test_exact_integer_products(0, 0, 17, 9, 64), T_GEMM.test_within_recursive_summation_error_bound]),
    ("tree_result_largest_first",
     "float* acc = f->stack[f->depth - 1].part;\n    for (int s = f->depth - 2; s >= 0; --s) {",
     "float* acc = f->stack[0].part;\n    for (int s = 1; s < f->depth; ++s) {",
     [T_TREE.test_non_power_of_two_remainder_folded_first]),
    ("tree_sequential_fold", "while (f->depth > 0 && f->stack[f->depth - 1].level == level)", "while (0)",
     [lambda: T_TREE.test_treefold_equals_recursive_doubling(8)]),
    ("tree_divides", "out[i] = f_mul(acc[i], rR);", "out[i] = f_div(acc[i], (float)R);",
     [lambda: T_TREE.test_average_is_reciprocal_multiply_not_division(3)]),
    ("replay_microbatch_unscaled", "for (int64_t i = 0; i < n; ++i) g[i] = f_add(g[i], f_mul(x[i], r_accum));",
     "for (int64_t i = 0; i < n; ++i) g[i] = f_add(g[i], x[i]);",
     [lambda: T_REPLAY.test_integer_gradients_give_the_exact_mean(2, 4, 2)]),
    ("replay_shard_divides", "for (int64_t i = 0; i < n; ++i) inner[i] = f_mul(inner[i], r_shard);",
     "for (int64_t i = 0; i < n; ++i) inner[i] = f_div(inner[i], (float)dp_shard);",
     [T_REPLAY.test_every_average_is_a_reciprocal_multiply]),
    ("replay_microbatch_major_buffers", "const float* x = grads[r * accum + k];", "const float* x = grads[k * N + r];",
     [T_REPLAY.test_buffers_are_rank_major_then_microbatch]),
    ("fold_push_skips_carry", "while ((pushed >> level) & 1) {", "while (0) {",
     [lambda: T_REPLAY.test_streaming_push_result_equals_treefold(6)]),
    ("adamw_eps_inside_root", "const float d = f_add(sq, eps);", "const float d = f_sqrt(f_add(vh, eps));",
     [T_ADAMW.test_first_step_closed_form, T_ADAMW.test_constant_gradient_trajectory]),
    ("adamw_no_bias_correction_m", "const float mh = f_mul(mn, s.r1);", "const float mh = mn;",
     [T_ADAMW.test_constant_gradient_trajectory, T_ADAMW.test_dyadic_case_is_exact]),
    ("adamw_wd_sign", "const float z = f_add(u, y);", "const float z = f_sub(u, y);",
     [T_ADAMW.test_first_step_closed_form, T_ADAMW.test_dyadic_case_is_exact]),
    ("adamw_moments_swapped", "Mo[i] = mn;\n        V[i] = vn;", "Mo[i] = vn;\n        V[i] = mn;",
     [T_ADAMW.test_dyadic_case_is_exact]),
    ("adamw_beta_power_off_by_one", "for (int64_t t = 1; t < step; ++t)", "for (int64_t t = 0; t < step; ++t)",
     [T_ADAMW.test_dyadic_case_is_exact, T_ADAMW.test_host_scalars]),
    ("hash_inner_depth", "sh_node(level + 32 * c0, (size_t)nc * 32, (uint64_t)j, depth,",
     "sh_node(level + 32 * c0, (size_t)nc * 32, (uint64_t)j, 1,", [lambda: T_HASH.test_tree_mode_matches_hashlib(16 * 16 * 1024 + 5)]),
    ("hash_no_last_leaf_flag", "(uint64_t)i, 0, i == leaves - 1,", "(uint64_t)i, 0, 0,",
     [lambda: T_HASH.test_tree_mode_matches_hashlib(1025)]),
    ("blake2b_rotation", "v[b] = rotr64(v[b] ^ v[c], 63);", "v[b] = rotr64(v[b] ^ v[c], 62);",
     [T_HASH.test_rfc7693_known_answer]),
    ("fma_double_rounding", "const double s = sum_round_to_odd((double)a * (double)b, (double)c);",
     "const double s = (double)a * (double)b + (double)c;",
     [lambda: T_FMA.test_no_double_rounding(1)]),
    ("fma_flush_before_rounding", "if (fabs(r24) < 0x1p-126)", "if (fabs(s) < 0x1p-126)",
     [T_FMA.test_flush_after_rounding_to_24_bits]),
    ("gemm_fma_unfused", "acc = f_fma(a, b, acc);", "acc = f_add(acc, f_mul(a, b));",
     [T_FMA.test_fused_witness]),
    ("bf16_truncates", "    if (dlo < dhi) r = lo;", "    if (1) r = lo;",
     [T_BF16.test_bf16_round_matches_torch]),
    ("norm_result_largest_first",
     "acc = val[depth - 1];\n        for (int d = depth - 2; d >= 0; --d) acc = f_add(acc, val[d]);",
     "acc = val[0];\n        for (int d = 1; d < depth; ++d) acc = f_add(acc, val[d]);",
     [T_BF16.test_fold_result_starts_from_the_smallest_block]),
    ("skipped_step_applies", "    if (apply) {\n        const int64_t t = st->step + 1;",
     "    if (1) {\n        const int64_t t = st->step + 1;",
     [T_BF16.test_spike_protocol_skips_five_steps_without_advancing_the_count]),
    ("spike_window_not_restarted", "norm > spike_threshold) st->skip_left = skip_steps;",
     "norm > spike_threshold && st->skip_left == 0) st->skip_left = skip_steps;",
     [T_BF16.test_spike_inside_the_window_starts_it_again]),
    ("clip_without_epsilon", "f_div(max_norm, f_add(norm, 1e-6f))", "f_div(max_norm, norm)",
     [lambda: T_BF16.test_clip_scales_every_element_by_the_coefficient(0.0205)]),
    ("no_flush", "_mm_setcsr((e.saved & ~0x6000u) | 0x8000u | 0x0040u | 0x1F80u);",
     "_mm_setcsr((e.saved & ~(0x6000u | 0x8000u | 0x0040u)) | 0x1F80u);",
     [T_FP32.test_subnormal_results_flush_with_sign, T_FP32.test_subnormal_operands_read_as_signed_zero]),
    # Flushing after rounding onto the subnormal grid (instead of the x86
    # unbounded-exponent rounding) differs at the smallest normal.
    ("flush_after_gradual_underflow", "static float f_mul(float a, float b) { return a * b; }",
     "static float f_mul(float a, float b) { unsigned c = _mm_getcsr(); _mm_setcsr(c & ~0x8040u); "
     "float r = a * b; _mm_setcsr(c); return fpclassify(r) == FP_SUBNORMAL ? copysignf(0.0f, r) : r; }",
     [T_FP32.test_tininess_is_decided_after_rounding_with_unbounded_exponent]),
    ("flush_before_rounding", "static float f_mul(float a, float b) { return a * b; }",
     "static float f_mul(float a, float b) { double e = (double)a * (double)b; "
     "return fabs(e) < 0x1p-126 ? copysignf(0.0f, (float)e) : a * b; }",
     [T_FP32.test_tininess_is_decided_after_rounding_with_unbounded_exponent]),
]


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name,find,repl,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(workdir, name, find, repl, pins):
    src = open(SRC).read()
    assert src.count(find) >= 1, f"mutation anchor not found: {find!r}"
    mutated = src.replace(find, repl, 1)
    cpath = os.path.join(workdir, f"{name}.c")
    with open(cpath, "w") as fh:
        fh.write(mutated)
    lib = os.path.join(workdir, f"lib{name}.so")
    subprocess.run(["gcc", *oracle_build.FLAGS, cpath, "-o", lib, "-lm"], check=True)
    with oracle.swap_library(lib):
        for pin in pins:
            with pytest.raises(AssertionError):
                pin()
