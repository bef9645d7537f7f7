// The BF16-parameter optimizer step: the pre-clip global gradient norm, the
// clip and spike decision, and the fused update.
//
// "OPEN-1B: A Fully Auditable Training Run": section 3.1 (parameters held in
// BF16), section 3.2 "Optimizer" (AdamW, gradients clipped to a global l2
// norm of 1.0) and "Optimizer-state precision" (the fused step widens the
// BF16 parameter and gradient to FP32, updates with FP32 moments and rounds
// the parameter to BF16 once), section 3.4.2 (five optimizer steps skipped
// when the pre-clip norm exceeds 5), Appendix A.1 (TreeFold, here the order
// of the norm's sum).
//
// Design for gfx950:
//  - The norm's sum S = TreeFold(g_0^2, ..., g_{n-1}^2) in index order.  For
//    terms >= +0 the fold equals one perfect pairwise tree over the terms
//    padded with +0 to a power of two (the fold's Result nests the blocks
//    from the smallest, and a padded subtree adds +0, which changes no value
//    that is not -0; squares and their sums are never -0).  So each
//    workgroup folds an aligned block of 4096 terms as a perfect tree - four
//    terms per lane, lane pairs by xor shuffles, then chunks and waves - and
//    the block sums are folded again by the same kernel until one value is
//    left: three launches for 1.2e9 terms, every load a coalesced 1 KB per
//    wave instruction.
//  - One thread then takes S to the norm and applies the clip and spike
//    rules to the caller's step record in device memory, so a whole step is
//    stream-ordered work with no host round trip.
//  - The update streams w (bf16), m, v (fp32) and g (fp32 or bf16) once,
//    four elements per thread, with the sixteen AdamW operations of the FP32
//    kernel in between; a skipped step exits before touching memory.
#include <hip/hip_runtime.h>

#include "device_ops.h"
#include "internal.h"
#include "repro.h"

namespace repro {
namespace {

constexpr int kNormBlock = 4096;  // terms folded by one workgroup

__device__ __forceinline__ float widen_bf16(uint32_t h) { return __uint_as_float((h & 0xFFFFu) << 16); }

// binary32 -> bf16, round to nearest, ties to even (carry into the exponent,
// and on to infinity past the largest bf16, as IEEE rounding does).  The
// input is a normal value or a zero (every result of the update is), so no
// flush is needed.
__device__ __forceinline__ uint32_t round_bf16(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// SRC 0: squares of binary32 terms; 1: squares of bf16 terms; 2: binary32
// terms as they are (block sums of an earlier pass).
template <int SRC>
__device__ __forceinline__ float4 load_terms(const void* src, int64_t e, int64_t len, bool vec) {
  float4 x;
  if (vec) {
    if constexpr (SRC == 1) {
      const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(src) + e);
      x = make_float4(widen_bf16(h.x), widen_bf16(h.x >> 16), widen_bf16(h.y), widen_bf16(h.y >> 16));
    } else {
      x = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + e);
    }
  } else {
    float t[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (e + k < len) {
        if constexpr (SRC == 1)
          t[k] = widen_bf16(static_cast<const uint16_t*>(src)[e + k]);
        else
          t[k] = static_cast<const float*>(src)[e + k];
      } else {
        t[k] = 0.0f;  // padding
      }
    }
    x = make_float4(t[0], t[1], t[2], t[3]);
  }
  if constexpr (SRC != 2) x = make_float4(mul_c(x.x, x.x), mul_c(x.y, x.y), mul_c(x.z, x.z), mul_c(x.w, x.w));
  return x;
}

// One workgroup (4 waves) folds terms [4096 b, 4096 b + 4096) of a length
// len sequence as a perfect pairwise tree and writes out[b].  Wave w takes
// [1024 w, 1024 w + 1024) as four chunks of 256 with lane l holding terms
// 4l .. 4l+3 (binary32 terms), or as two chunks of 512 with lane l holding
// 8l .. 8l+7 (bf16 terms); either way one wave instruction loads 1 KB.
template <int SRC>
__global__ __launch_bounds__(256) void k_norm_fold(const void* __restrict__ src, int64_t len, bool aligned,
                                                   float* __restrict__ out) {
  const int64_t b = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t base = b * kNormBlock + wave * 1024;
  const bool vec = aligned && (b + 1) * kNormBlock <= len;
  float wsum;
  if constexpr (SRC == 1) {
    // bf16 terms: two chunks of 512, lane l holding terms 8l .. 8l+7 (one
    // 16-byte load); the same perfect tree, levels 1-3 in the lane and 4-9
    // across lanes, then the two chunks.
    float chunk[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t e = base + j * 512 + 8 * lane;
      float4 x, y;
      if (vec) {
        const uint4 h = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + e);
        x = make_float4(widen_bf16(h.x), widen_bf16(h.x >> 16), widen_bf16(h.y), widen_bf16(h.y >> 16));
        y = make_float4(widen_bf16(h.z), widen_bf16(h.z >> 16), widen_bf16(h.w), widen_bf16(h.w >> 16));
        x = make_float4(mul_c(x.x, x.x), mul_c(x.y, x.y), mul_c(x.z, x.z), mul_c(x.w, x.w));
        y = make_float4(mul_c(y.x, y.x), mul_c(y.y, y.y), mul_c(y.z, y.z), mul_c(y.w, y.w));
      } else {
        x = load_terms<1>(src, e, len, false);
        y = load_terms<1>(src, e + 4, len, false);
      }
      float s = add_c(add_c(add_c(x.x, x.y), add_c(x.z, x.w)), add_c(add_c(y.x, y.y), add_c(y.z, y.w)));
#pragma unroll
      for (int k = 1; k < 64; k <<= 1) s = add_c(s, __shfl_xor(s, k, 64));
      chunk[j] = s;
    }
    wsum = add_c(chunk[0], chunk[1]);
  } else {
    float chunk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 x = load_terms<SRC>(src, base + j * 256 + 4 * lane, len, vec);
      float s = add_c(add_c(x.x, x.y), add_c(x.z, x.w));
      // Levels 3..8: lane l and lane l ^ k hold neighbouring blocks; both
      // form the same sum (IEEE addition commutes bit for bit).
#pragma unroll
      for (int k = 1; k < 64; k <<= 1) s = add_c(s, __shfl_xor(s, k, 64));
      chunk[j] = s;
    }
    wsum = add_c(add_c(chunk[0], chunk[1]), add_c(chunk[2], chunk[3]));
  }
  __shared__ float wave_sum[4];
  if (lane == 0) wave_sum[wave] = wsum;
  __syncthreads();
  if (threadIdx.x == 0) out[b] = add_c(add_c(wave_sum[0], wave_sum[1]), add_c(wave_sum[2], wave_sum[3]));
}

// One thread: S -> norm, then (with a step record) the spike and clip
// rules and the host scalars of an applied step, in binary32 under the
// contract, exactly as a host would compute them.
__global__ __launch_bounds__(64) void k_norm_finish(OptHeader* hdr, int64_t n, float* out2, repro_step_state* st,
                                                    float beta1, float beta2, float max_norm,
                                                    float spike_threshold, int skip_steps) {
  if (threadIdx.x != 0) return;
  const float S = n == 0 ? 0.0f : hdr->sumsq;
  const float norm = sqrt_c(S);
  hdr->sumsq = S;
  hdr->norm = norm;
  if (out2 != nullptr) {
    out2[0] = norm;
    out2[1] = S;
  }
  if (st == nullptr) return;
  st->grad_norm = norm;
  if (spike_threshold > 0.0f && norm > spike_threshold) st->skip_left = skip_steps;
  int apply = 1;
  if (st->skip_left > 0) {
    apply = 0;
    st->skip_left -= 1;
  }
  float coef = 1.0f;
  if (max_norm > 0.0f) {
    const float c = div_c(max_norm, add_c(norm, 1e-6f));
    if (c < 1.0f) coef = c;
  }
  st->clip_coef = coef;
  st->applied = apply;
  hdr->apply = apply;
  hdr->coef = coef;
  if (apply) {
    const int64_t t = st->step + 1;
    const float p1 = t == 1 ? beta1 : mul_c(st->beta1_pow, beta1);
    const float p2 = t == 1 ? beta2 : mul_c(st->beta2_pow, beta2);
    hdr->c1 = sub_c(1.0f, beta1);
    hdr->c2 = sub_c(1.0f, beta2);
    hdr->r1 = div_c(1.0f, sub_c(1.0f, p1));
    hdr->r2 = div_c(1.0f, sub_c(1.0f, p2));
    st->step = t;
    st->beta1_pow = p1;
    st->beta2_pow = p2;
  }
}

__device__ __forceinline__ AdamwScalars scalars_of(const OptHeader* hdr, float lr, float beta1, float beta2,
                                                   float eps, float wd) {
  AdamwScalars s;
  s.lr = lr;
  s.beta1 = beta1;
  s.beta2 = beta2;
  s.eps = eps;
  s.wd = wd;
  s.c1 = hdr->c1;
  s.c2 = hdr->c2;
  s.r1 = hdr->r1;
  s.r2 = hdr->r2;
  return s;
}

__device__ __forceinline__ float clip_grad(float g, float coef) { return coef < 1.0f ? mul_c(g, coef) : g; }

// Four elements per thread over an exact grid of n/4 threads.  GBF16: the
// gradient is bf16 (else binary32).
template <bool GBF16>
__global__ __launch_bounds__(kStreamLanes) void k_adamw_bf16_v4(uint2* __restrict__ w4, float4* __restrict__ m4,
                                                       float4* __restrict__ v4, const void* __restrict__ g,
                                                       int64_t n4, const OptHeader* __restrict__ hdr, float lr,
                                                       float beta1, float beta2, float eps, float wd) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4 || hdr->apply == 0) return;
  const AdamwScalars s = scalars_of(hdr, lr, beta1, beta2, eps, wd);
  const float coef = hdr->coef;
  const uint2 wh = w4[i];
  float4 m = ld_nt(m4 + i);
  float4 v = ld_nt(v4 + i);
  float4 gg;
  if constexpr (GBF16) {
    const uint2 gh = static_cast<const uint2*>(g)[i];
    gg = make_float4(widen_bf16(gh.x), widen_bf16(gh.x >> 16), widen_bf16(gh.y), widen_bf16(gh.y >> 16));
  } else {
    gg = ld_nt(static_cast<const float4*>(g) + i);
  }
  float w0 = widen_bf16(wh.x), w1 = widen_bf16(wh.x >> 16), w2 = widen_bf16(wh.y), w3 = widen_bf16(wh.y >> 16);
  adamw_elem(w0, m.x, v.x, clip_grad(gg.x, coef), s);
  adamw_elem(w1, m.y, v.y, clip_grad(gg.y, coef), s);
  adamw_elem(w2, m.z, v.z, clip_grad(gg.z, coef), s);
  adamw_elem(w3, m.w, v.w, clip_grad(gg.w, coef), s);
  w4[i] = make_uint2(round_bf16(w0) | (round_bf16(w1) << 16), round_bf16(w2) | (round_bf16(w3) << 16));
  st_nt(m, m4 + i);
  st_nt(v, v4 + i);
}

template <bool GBF16>
__global__ __launch_bounds__(256) void k_adamw_bf16_s(uint16_t* __restrict__ w, float* __restrict__ m,
                                                      float* __restrict__ v, const void* __restrict__ g,
                                                      int64_t first, int64_t n, const OptHeader* __restrict__ hdr,
                                                      float lr, float beta1, float beta2, float eps, float wd) {
  if (hdr->apply == 0) return;
  const AdamwScalars s = scalars_of(hdr, lr, beta1, beta2, eps, wd);
  const float coef = hdr->coef;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float gi = GBF16 ? widen_bf16(static_cast<const uint16_t*>(g)[i]) : static_cast<const float*>(g)[i];
    float wi = widen_bf16(w[i]), mi = m[i], vi = v[i];
    adamw_elem(wi, mi, vi, clip_grad(gi, coef), s);
    w[i] = (uint16_t)round_bf16(wi);
    m[i] = mi;
    v[i] = vi;
  }
}

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

void plan_grad_norm(int64_t n, NormPlan* plan) {
  plan->passes = 0;
  int64_t off = kOptHeaderBytes;
  int64_t len = n;
  while (len > 0) {
    const int64_t outs = (len + kNormBlock - 1) / kNormBlock;
    plan->len[plan->passes] = len;
    plan->out_offset[plan->passes] = outs == 1 ? -1 : off;  // the last pass writes the header
    ++plan->passes;
    if (outs == 1) break;
    off += ((outs * 4 + 255) / 256) * 256;
    len = outs;
  }
  plan->total_bytes = off;
}

hipError_t launch_grad_norm(const void* g, int dtype, int64_t n, uint8_t* ws, const NormPlan& plan, float* out2,
                            repro_step_state* st, const StepRule& rule, hipStream_t stream) {
  OptHeader* hdr = reinterpret_cast<OptHeader*>(ws);
  const void* src = g;
  for (int p = 0; p < plan.passes; ++p) {
    const int64_t len = plan.len[p];
    const int64_t grid = (len + kNormBlock - 1) / kNormBlock;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    float* out = plan.out_offset[p] < 0 ? &hdr->sumsq : reinterpret_cast<float*>(ws + plan.out_offset[p]);
    if (p == 0 && dtype == 1) {
      hipLaunchKernelGGL(k_norm_fold<1>, dim3((unsigned)grid), dim3(256), 0, stream, src, len,
                         aligned_to(src, 16), out);
    } else if (p == 0) {
      hipLaunchKernelGGL(k_norm_fold<0>, dim3((unsigned)grid), dim3(256), 0, stream, src, len,
                         aligned_to(src, 16), out);
    } else {
      hipLaunchKernelGGL(k_norm_fold<2>, dim3((unsigned)grid), dim3(256), 0, stream, src, len, true, out);
    }
    src = out;
  }
  hipLaunchKernelGGL(k_norm_finish, dim3(1), dim3(64), 0, stream, hdr, n, out2, st, rule.beta1, rule.beta2,
                     rule.max_norm, rule.spike_threshold, rule.skip_steps);
  return hipGetLastError();
}

hipError_t launch_adamw_bf16(uint16_t* w, float* m, float* v, const void* g, int dtype, int64_t n, const uint8_t* ws,
                             float lr, float beta1, float beta2, float eps, float wd, hipStream_t stream) {
  const OptHeader* hdr = reinterpret_cast<const OptHeader*>(ws);
  const bool vec = aligned_to(w, 8) && aligned_to(m, 16) && aligned_to(v, 16) && aligned_to(g, dtype == 1 ? 8 : 16);
  const int64_t n4 = vec ? n / 4 : 0;
  if (n4 > 0) {
    const int64_t grid = (n4 + kStreamLanes - 1) / kStreamLanes;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (dtype == 1)
      hipLaunchKernelGGL(k_adamw_bf16_v4<true>, dim3((unsigned)grid), dim3(kStreamLanes), 0, stream,
                         reinterpret_cast<uint2*>(w), reinterpret_cast<float4*>(m), reinterpret_cast<float4*>(v), g,
                         n4, hdr, lr, beta1, beta2, eps, wd);
    else
      hipLaunchKernelGGL(k_adamw_bf16_v4<false>, dim3((unsigned)grid), dim3(kStreamLanes), 0, stream,
                         reinterpret_cast<uint2*>(w), reinterpret_cast<float4*>(m), reinterpret_cast<float4*>(v), g,
                         n4, hdr, lr, beta1, beta2, eps, wd);
  }
  const int64_t first = 4 * n4;
  if (first < n) {
    int64_t grid = (n - first + 255) / 256;
    if (grid > (int64_t(1) << 20)) grid = int64_t(1) << 20;
    if (dtype == 1)
      hipLaunchKernelGGL(k_adamw_bf16_s<true>, dim3((unsigned)grid), dim3(256), 0, stream, w, m, v, g, first, n,
                         hdr, lr, beta1, beta2, eps, wd);
    else
      hipLaunchKernelGGL(k_adamw_bf16_s<false>, dim3((unsigned)grid), dim3(256), 0, stream, w, m, v, g, first, n,
                         hdr, lr, beta1, beta2, eps, wd);
  }
  return hipGetLastError();
}

}  // namespace repro
