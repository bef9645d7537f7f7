// Device helpers shared by the element-wise kernels: one binary32 contract
// operation each, and 16-byte streaming loads and stores.  Every file that
// includes this is built with -fgpu-flush-denormals-to-zero and
// -ffp-contract=off (see build.py), so each helper is one IEEE operation
// followed by the x86-style flush of the hardware mode, never fused.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace repro {
namespace {

// One binary32 operation each (the hardware mode applies the flush rule).
__device__ __forceinline__ float add_c(float a, float b) { return a + b; }
__device__ __forceinline__ float sub_c(float a, float b) { return a - b; }
__device__ __forceinline__ float mul_c(float a, float b) { return a * b; }
__device__ __forceinline__ float div_c(float a, float b) { return a / b; }
__device__ __forceinline__ float sqrt_c(float a) { return __builtin_sqrtf(a); }

// Workgroup size of the streaming kernels (one 16-byte vector per lane, an
// exact grid): one wave.  Measured on MI355X against 256 lanes, with the
// same bits: AdamW 5.39 vs 5.80 ms, the replay 1.53 vs 1.65-1.74 ms, the
// tree reduce 99 vs 104 us (median), the BF16 update 3-5% and a plain copy
// 6.67 vs 6.42 TB/s; 128 and 512 lanes fell in between.
constexpr int kStreamLanes = 64;

// Streaming 16-byte accesses that bypass cache retention (nontemporal).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float4 v, float4* p) {
  f4v u = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(u, reinterpret_cast<f4v*>(p));
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(add_c(a.x, b.x), add_c(a.y, b.y), add_c(a.z, b.z), add_c(a.w, b.w));
}
__device__ __forceinline__ float4 mul4s(float4 a, float s) {
  return make_float4(mul_c(a.x, s), mul_c(a.y, s), mul_c(a.z, s), mul_c(a.w, s));
}
__device__ __forceinline__ float add_v(float a, float b) { return add_c(a, b); }
__device__ __forceinline__ float4 add_v(float4 a, float4 b) { return add4(a, b); }
__device__ __forceinline__ float mul_vs(float a, float s) { return mul_c(a, s); }
__device__ __forceinline__ float4 mul_vs(float4 a, float s) { return mul4s(a, s); }

// AdamW ("OPEN-1B: A Fully Auditable Training Run", section 3.2
// "Optimizer"): the sixteen operations in their declared order, each one
// rounding, with the host scalars c1 = 1 - beta1, c2 = 1 - beta2 and the
// bias-correction reciprocals r1, r2.
__device__ __forceinline__ void adamw_elem(float& w, float& m, float& v, float g, const AdamwScalars& s) {
  const float m1 = mul_c(s.beta1, m);
  const float m2 = mul_c(s.c1, g);
  const float mn = add_c(m1, m2);
  const float q = mul_c(g, g);
  const float v1 = mul_c(s.beta2, v);
  const float v2 = mul_c(s.c2, q);
  const float vn = add_c(v1, v2);
  const float mh = mul_c(mn, s.r1);
  const float vh = mul_c(vn, s.r2);
  const float sq = sqrt_c(vh);
  const float d = add_c(sq, s.eps);
  const float u = div_c(mh, d);
  const float y = mul_c(s.wd, w);
  const float z = add_c(u, y);
  const float t = mul_c(s.lr, z);
  const float wn = sub_c(w, t);
  w = wn;
  m = mn;
  v = vn;
}

}  // namespace
}  // namespace repro
