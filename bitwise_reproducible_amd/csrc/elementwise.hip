// Element-wise reproducible kernels: the TreeFold replica reduction and the
// fused AdamW step, plus the diagnostic single-operation kernel.
//
// Numeric contract ("OPEN-1B: A Fully Auditable Training Run", section 2.1
// and Table 1): this file is built with -fgpu-flush-denormals-to-zero, so the
// kernel descriptors select the fp32 mode that flushes subnormal operands and
// results.  Measured on gfx950, that flush is the x86 FTZ/DAZ rule the
// oracle uses (a result is zeroed when, rounded to 24 bits with an unbounded
// exponent, it is below 2^-126), bit for bit.  -ffp-contract=off keeps every
// multiply and add separate (section 2.1 "Fused multiply-add").  Division
// and square root use the compiler's correctly rounded sequences; the tests
// check them against the oracle, the square root over all 2^31 non-negative
// inputs.
#include <hip/hip_runtime.h>

#include <array>
#include <utility>

#include "device_ops.h"
#include "internal.h"

namespace repro {
namespace {

// ---------------------------------------------------------------------------
// TreeFold (Appendix A.1, Algorithm 2), unrolled at compile time for a fixed
// replica count R.  Pushing replicas 0..R-1 in order leaves one block per set
// bit of R on the stack: the block of the highest bit covers the lowest
// replicas.  A block of 2^b replicas is the balanced pairwise tree that Push
// builds by carrying (lower half on the left).  Result starts from the block
// of the lowest set bit and adds the blocks of the higher set bits in
// ascending order.

// Sum of replicas [LO, LO + SIZE), SIZE a power of two.
template <int LO, int SIZE, typename V>
__device__ __forceinline__ V fold_block(const V* x) {
  if constexpr (SIZE == 1) {
    return x[LO];
  } else {
    return add_v(fold_block<LO, SIZE / 2>(x), fold_block<LO + SIZE / 2, SIZE / 2>(x));
  }
}

// First replica of the block that belongs to bit BIT of R.
template <int R, int BIT>
constexpr int block_start() {
  return R & ~((2 << BIT) - 1);
}

template <int R, int BIT, typename V>
__device__ __forceinline__ V fold_rest(V acc, const V* x) {
  if constexpr (BIT >= 7) {
    return acc;
  } else {
    if constexpr (((R >> BIT) & 1) != 0) {
      acc = add_v(acc, fold_block<block_start<R, BIT>(), (1 << BIT)>(x));
    }
    return fold_rest<R, BIT + 1>(acc, x);
  }
}

template <int R>
constexpr int lowest_bit() {
  int b = 0;
  while (((R >> b) & 1) == 0) ++b;
  return b;
}

template <int R, typename V>
__device__ __forceinline__ V tree_fold(const V* x) {
  constexpr int lb = lowest_bit<R>();
  V acc = fold_block<block_start<R, lb>(), (1 << lb)>(x);
  return fold_rest<R, lb + 1>(acc, x);
}

static_assert(REPRO_MAX_REPLICAS <= 127, "fold_rest walks bits 0..6");

// One 16-byte vector per replica per thread (the grid covers all n/4
// vectors; measured on MI355X this shape streams faster than a grid-stride
// loop).  AVG selects the multiply by fl(1/R) at compile time.
template <int R, bool AVG>
__global__ __launch_bounds__(kStreamLanes) void k_tree_reduce_v4(ReplicaPtrs reps, float4* __restrict__ out, int64_t n4,
                                                         float rR) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  float4 x[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = ld_nt(reinterpret_cast<const float4*>(reps.p[r]) + i);
  float4 s = tree_fold<R>(x);
  if constexpr (AVG) s = mul4s(s, rR);
  st_nt(s, out + i);
}

// The same with a grid-stride loop over a capped grid (launch-shape variant).
template <int R>
__global__ __launch_bounds__(256) void k_tree_reduce_v4_strided(ReplicaPtrs reps, float4* __restrict__ out,
                                                                 int64_t n4, float rR, int average) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    float4 x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = ld_nt(reinterpret_cast<const float4*>(reps.p[r]) + i);
    float4 s = tree_fold<R>(x);
    if (average) s = mul4s(s, rR);
    st_nt(s, out + i);
  }
}

// Scalar elements [first, n).
template <int R>
__global__ __launch_bounds__(256) void k_tree_reduce_s(ReplicaPtrs reps, float* __restrict__ out, int64_t first,
                                                        int64_t n, float rR, int average) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float x[R];
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = reps.p[r][i];
    float s = tree_fold<R>(x);
    if (average) s = mul_c(s, rR);
    out[i] = s;
  }
}

using V4Fn = void (*)(ReplicaPtrs, float4*, int64_t, float);
using V4SFn = void (*)(ReplicaPtrs, float4*, int64_t, float, int);
using SFn = void (*)(ReplicaPtrs, float*, int64_t, int64_t, float, int);

template <bool AVG, int... Rs>
constexpr auto make_v4_table(std::integer_sequence<int, Rs...>) {
  return std::array<V4Fn, sizeof...(Rs)>{{&k_tree_reduce_v4<Rs + 1, AVG>...}};
}
template <int... Rs>
constexpr auto make_v4s_table(std::integer_sequence<int, Rs...>) {
  return std::array<V4SFn, sizeof...(Rs)>{{&k_tree_reduce_v4_strided<Rs + 1>...}};
}
template <int... Rs>
constexpr auto make_s_table(std::integer_sequence<int, Rs...>) {
  return std::array<SFn, sizeof...(Rs)>{{&k_tree_reduce_s<Rs + 1>...}};
}

const auto kV4Table = make_v4_table<false>(std::make_integer_sequence<int, REPRO_MAX_REPLICAS>{});
const auto kV4AvgTable = make_v4_table<true>(std::make_integer_sequence<int, REPRO_MAX_REPLICAS>{});
const auto kV4StridedTable = make_v4s_table(std::make_integer_sequence<int, REPRO_MAX_REPLICAS>{});
const auto kSTable = make_s_table(std::make_integer_sequence<int, REPRO_MAX_REPLICAS>{});

int64_t grid_for(int64_t items, int threads, int64_t cap) {
  int64_t g = (items + threads - 1) / threads;
  if (g < 1) g = 1;
  return g < cap ? g : cap;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// AdamW (section 3.2 "Optimizer"): adamw_elem in device_ops.h.
__global__ __launch_bounds__(kStreamLanes) void k_adamw_v4(float4* __restrict__ w4, float4* __restrict__ m4,
                                                   float4* __restrict__ v4, const float4* __restrict__ g4,
                                                   int64_t n4, AdamwScalars s) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  float4 w = ld_nt(w4 + i);
  float4 m = ld_nt(m4 + i);
  float4 v = ld_nt(v4 + i);
  const float4 g = ld_nt(g4 + i);
  adamw_elem(w.x, m.x, v.x, g.x, s);
  adamw_elem(w.y, m.y, v.y, g.y, s);
  adamw_elem(w.z, m.z, v.z, g.z, s);
  adamw_elem(w.w, m.w, v.w, g.w, s);
  st_nt(w, w4 + i);
  st_nt(m, m4 + i);
  st_nt(v, v4 + i);
}

__global__ __launch_bounds__(256) void k_adamw_s(float* __restrict__ w, float* __restrict__ m,
                                                  float* __restrict__ v, const float* __restrict__ g,
                                                  int64_t first, int64_t n, AdamwScalars s) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float wi = w[i], mi = m[i], vi = v[i];
    adamw_elem(wi, mi, vi, g[i], s);
    w[i] = wi;
    m[i] = mi;
    v[i] = vi;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fp32_ops(int op, const float* __restrict__ a,
                                                   const float* __restrict__ b, float* __restrict__ out,
                                                   int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float x = a[i];
    const float y = b[i];
    float r;
    switch (op) {
      case 0: r = add_c(x, y); break;
      case 1: r = sub_c(x, y); break;
      case 2: r = mul_c(x, y); break;
      case 3: r = div_c(x, y); break;
      default: r = sqrt_c(x); break;
    }
    out[i] = r;
  }
}

}  // namespace

hipError_t launch_tree_reduce(const ReplicaPtrs& reps, int R, int64_t n, float* out, int average, float rR,
                              int variant, hipStream_t stream) {
  bool vec = variant != 1 && aligned16(out);
  for (int r = 0; r < R; ++r) vec = vec && aligned16(reps.p[r]);
  const int64_t n4 = vec ? n / 4 : 0;
  if (n4 > 0) {
    if (variant == 2) {
      hipLaunchKernelGGL(kV4StridedTable[R - 1], dim3((unsigned)grid_for(n4, 64, 1024)), dim3(64), 0, stream, reps,
                         reinterpret_cast<float4*>(out), n4, rR, average);
    } else {
      const int64_t grid = (n4 + kStreamLanes - 1) / kStreamLanes;
      if (grid > 0x7fffffff) return hipErrorInvalidValue;
      hipLaunchKernelGGL((average ? kV4AvgTable : kV4Table)[R - 1], dim3((unsigned)grid), dim3(kStreamLanes), 0,
                         stream,
                         reps, reinterpret_cast<float4*>(out), n4, rR);
    }
  }
  const int64_t first = n4 * 4;
  if (first < n) {
    const int64_t grid = grid_for(n - first, 256, int64_t(1) << 20);
    hipLaunchKernelGGL(kSTable[R - 1], dim3((unsigned)grid), dim3(256), 0, stream, reps, out, first, n, rR,
                       average);
  }
  return hipGetLastError();
}

hipError_t launch_adamw(float* state, const float* grad, int64_t n, const AdamwScalars& s, int variant,
                        hipStream_t stream) {
  return launch_adamw_ptrs(state, state + n, state + 2 * n, grad, n, s, variant, stream);
}

hipError_t launch_adamw_ptrs(float* w, float* m, float* v, const float* grad, int64_t n, const AdamwScalars& s,
                             int variant, hipStream_t stream) {
  const bool vec = variant != 1 && aligned16(w) && aligned16(m) && aligned16(v) && aligned16(grad);
  const int64_t n4 = vec ? n / 4 : 0;
  if (n4 > 0) {
    const int64_t grid = (n4 + kStreamLanes - 1) / kStreamLanes;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_adamw_v4, dim3((unsigned)grid), dim3(kStreamLanes), 0, stream, reinterpret_cast<float4*>(w),
                       reinterpret_cast<float4*>(m), reinterpret_cast<float4*>(v),
                       reinterpret_cast<const float4*>(grad), n4, s);
  }
  const int64_t first = n4 * 4;
  if (first < n) {
    const int64_t grid = grid_for(n - first, 256, int64_t(1) << 20);
    hipLaunchKernelGGL(k_adamw_s, dim3((unsigned)grid), dim3(256), 0, stream, w, m, v, grad, first, n, s);
  }
  return hipGetLastError();
}

hipError_t launch_fp32_ops(int op, const float* a, const float* b, float* out, int64_t n,
                                hipStream_t stream) {
  const int64_t grid = grid_for(n, 256, int64_t(1) << 20);
  hipLaunchKernelGGL(k_fp32_ops, dim3((unsigned)grid), dim3(256), 0, stream, op, a, b, out, n);
  return hipGetLastError();
}

}  // namespace repro
