// The fused multiply-add convention, one operation per element, on the units
// that can carry a fused chain: the VALU (v_fma_f32) and the matrix cores
// (the K = 1 instructions v_mfma_f32_{32x32x1_2b, 16x16x1_4b, 4x4x1_16b}_f32
// with the chain value as the C operand).
//
// The pages keep multiply and add unfused ("OPEN-1B: A Fully Auditable
// Training Run", section 2.1 "Fused multiply-add"); the fused chain is a
// declared alternative: fl(a*b + c) rounded once under the subnormal rule of
// section 2.1 ("Subnormals").  These kernels exist so that the directed
// tests can check each unit's single step against that definition on chosen
// operands (flush boundary, ties, cancellation, signed zeros) before any
// GEMM is built on it.
//
// Matrix-core forms.  The instructions with K = 1 compute, for each of
// their independent S x S blocks b, D[i][j] = C[i][j] + A[i] * B[j]; lane
// S*b + i supplies A[i] and B[i] of block b.  Element t of a 64-element group
// goes to a block diagonal: lane t supplies a_t and b_t, and C[i][i] = c_t of
// block t / S, so the diagonal result is a_t * b_t + c_t.  Each lane holding a
// diagonal entry reads its c and writes its result directly from and to
// memory, so no cross-lane moves are needed.  Where D[i][j] of block b lives
// (lane, register r):
//   v_mfma_f32_32x32x1_2b_f32 (2 blocks):  lane j + 32 * ((i / 4) % 2),
//                                          r = 16 b + 4 (i / 8) + i % 4
//   v_mfma_f32_16x16x1_4b_f32 (4 blocks):  lane j + 16 (i / 4), r = 4 b + i % 4
//   v_mfma_f32_4x4x1_16b_f32 (16 blocks):  lane 4 b + j,        r = i
#include <hip/hip_runtime.h>

#include "internal.h"

namespace repro {
namespace {

typedef float floatx32 __attribute__((ext_vector_type(32)));

__global__ __launch_bounds__(256) void k_fma_valu(const float* a, const float* b,
                                                  const float* c, float* out,
                                                  int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = __builtin_fmaf(a[i], b[i], c[i]);
}

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int S>
struct MfmaK1;

template <>
struct MfmaK1<32> {
  static constexpr int kRegs = 32;
  typedef floatx32 V;
  static __device__ V step(float a, float b, V c) { return __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, c, 0, 0, 0); }
  static __device__ void place(int lane, int r, int& blk, int& i, int& j) {
    blk = r >> 4;
    const int rr = r & 15;
    i = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
    j = lane & 31;
  }
};

template <>
struct MfmaK1<16> {
  static constexpr int kRegs = 16;
  typedef floatx16 V;
  static __device__ V step(float a, float b, V c) { return __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, c, 0, 0, 0); }
  static __device__ void place(int lane, int r, int& blk, int& i, int& j) {
    blk = r >> 2;
    i = 4 * (lane >> 4) + (r & 3);
    j = lane & 15;
  }
};

template <>
struct MfmaK1<4> {
  static constexpr int kRegs = 4;
  typedef floatx4 V;
  static __device__ V step(float a, float b, V c) { return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0); }
  static __device__ void place(int lane, int r, int& blk, int& i, int& j) {
    blk = lane >> 2;
    i = r;
    j = lane & 3;
  }
};

template <int S>
__global__ __launch_bounds__(256) void k_fma_mfma(const float* a, const float* b, const float* c, float* out,
                                                  int64_t n) {
  using U = MfmaK1<S>;
  const int lane = threadIdx.x & 63;
  const int64_t groups = (n + 63) / 64;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t g = wave0; g < groups; g += wstride) {  // uniform across the wave
    const int64_t base = g * 64;
    const float av = base + lane < n ? a[base + lane] : 0.0f;
    const float bv = base + lane < n ? b[base + lane] : 0.0f;
    typename U::V cm;
#pragma unroll
    for (int r = 0; r < U::kRegs; ++r) {
      int blk, i, j;
      U::place(lane, r, blk, i, j);
      const int64_t t = base + S * blk + i;
      cm[r] = (i == j && t < n) ? c[t] : 0.0f;
    }
    const typename U::V d = U::step(av, bv, cm);
#pragma unroll
    for (int r = 0; r < U::kRegs; ++r) {
      int blk, i, j;
      U::place(lane, r, blk, i, j);
      const int64_t t = base + S * blk + i;
      if (i == j && t < n) out[t] = d[r];
    }
  }
}

}  // namespace

hipError_t launch_fp32_fma(int unit, const float* a, const float* b, const float* c, float* out, int64_t n,
                           hipStream_t stream) {
  const int64_t items = unit == 0 ? n : (n + 63) / 64 * 64;
  int64_t grid = (items + 255) / 256;
  if (grid > (int64_t(1) << 20)) grid = int64_t(1) << 20;
  switch (unit) {
    case 0: hipLaunchKernelGGL(k_fma_valu, dim3((unsigned)grid), dim3(256), 0, stream, a, b, c, out, n); break;
    case 1: hipLaunchKernelGGL(k_fma_mfma<32>, dim3((unsigned)grid), dim3(256), 0, stream, a, b, c, out, n); break;
    case 2: hipLaunchKernelGGL(k_fma_mfma<16>, dim3((unsigned)grid), dim3(256), 0, stream, a, b, c, out, n); break;
    case 3: hipLaunchKernelGGL(k_fma_mfma<4>, dim3((unsigned)grid), dim3(256), 0, stream, a, b, c, out, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace repro
