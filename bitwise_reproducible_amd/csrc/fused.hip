// The fused multiply-add convention, one operation per element, on the two
// units that can carry a fused chain: the VALU (v_fma_f32) and the matrix
// cores (v_mfma_f32_32x32x1_2b_f32 with the chain value as the C operand).
//
// The pages keep multiply and add unfused ("OPEN-1B: A Fully Auditable
// Training Run", section 2.1 "Fused multiply-add"); the fused chain is a
// declared alternative: fl(a*b + c) rounded once under the subnormal rule of
// section 2.1 ("Subnormals").  These kernels exist so that the directed
// tests can check each unit's single step against that definition on chosen
// operands (flush boundary, ties, cancellation, signed zeros) before any
// GEMM is built on it.
//
// Matrix-core form.  For each block b = 0, 1 the instruction computes
// D[i][j] = C[i][j] + A[i] * B[j] (K = 1), with A[i] and B[j] supplied by
// lane 32b + i and lane 32b + j, and D[i][j] of block b held by lane
// j + 32 * ((i / 4) % 2) in register 16b + 4 * (i / 8) + i % 4.  Element t of
// a 64-element group goes to the diagonal: A = a_t and B = b_t from lane t,
// C[i][i] = c_t; the diagonal result is a_t * b_t + c_t.  Each lane holding a
// diagonal entry reads its c and writes its result directly from and to
// memory, so no cross-lane moves are needed.
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

__global__ __launch_bounds__(256) void k_fma_mfma(const float* a, const float* b,
                                                  const float* c, float* out,
                                                  int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t groups = (n + 63) / 64;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t wstride = ((int64_t)gridDim.x * blockDim.x) >> 6;
  const int j = lane & 31;
  // Lanes whose column j also has the row i = j in their half hold a
  // diagonal entry of each block.
  const bool diag = ((j >> 2) & 1) == (lane >> 5);
  for (int64_t g = wave0; g < groups; g += wstride) {  // uniform across the wave
    const int64_t base = g * 64;
    const float av = base + lane < n ? a[base + lane] : 0.0f;
    const float bv = base + lane < n ? b[base + lane] : 0.0f;
    floatx32 cm;
#pragma unroll
    for (int r = 0; r < 32; ++r) cm[r] = 0.0f;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int rr = r & 15;
      const int i = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
      const int64_t t = base + 32 * (r >> 4) + i;
      if (diag && i == j && t < n) cm[r] = c[t];
    }
    const floatx32 d = __builtin_amdgcn_mfma_f32_32x32x1f32(av, bv, cm, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int rr = r & 15;
      const int i = 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
      const int64_t t = base + 32 * (r >> 4) + i;
      if (diag && i == j && t < n) out[t] = d[r];
    }
  }
}

}  // namespace

hipError_t launch_fp32_fma(int unit, const float* a, const float* b, const float* c, float* out, int64_t n,
                           hipStream_t stream) {
  const int64_t items = unit == 0 ? n : (n + 63) / 64 * 64;
  int64_t grid = (items + 255) / 256;
  if (grid > (int64_t(1) << 20)) grid = int64_t(1) << 20;
  if (unit == 0)
    hipLaunchKernelGGL(k_fma_valu, dim3((unsigned)grid), dim3(256), 0, stream, a, b, c, out, n);
  else
    hipLaunchKernelGGL(k_fma_mfma, dim3((unsigned)grid), dim3(256), 0, stream, a, b, c, out, n);
  return hipGetLastError();
}

}  // namespace repro
