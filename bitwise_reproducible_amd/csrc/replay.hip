// The audit replay of one step's gradient reduction, and TreeFold as a
// streaming interface.
//
// "OPEN-1B: A Fully Auditable Training Run", section 6 (Algorithm 1) and
// Appendix A.1-A.3 (Algorithm 2, reciprocal averages).  For N = dp_replicate
// x dp_shard virtual ranks in mesh order (r = rep * dp_shard + shard), each
// with `accum` microbatch gradients:
//   g_r = 0;  g_r = g_r + grad_k * fl(1/accum)      (microbatches in order)
//   inner = g_0;  inner = inner + g_s                 (shards ascending)
//   fold.Push(inner * fl(1/dp_shard))                 (once per replica)
//   out = fold.Result() * fl(1/dp_replicate)
//
// Design for gfx950: the whole algorithm runs per element in one pass over
// the N * accum gradient buffers, so every byte is read once and the output
// written once (HBM-bound, like the plain tree reduce).  A thread owns one
// 16-byte vector; the fold's level slots (at most 7 for 64 replicas) live in
// registers, indexed only by unrolled compile-time levels under uniform
// predicates, so nothing spills to scratch.  No atomics, no cross-lane sums.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_ops.h"
#include "internal.h"

namespace repro {
namespace {

constexpr int kLevels = kFoldSlots;

template <bool VEC>
using Elem = typename std::conditional<VEC, float4, float>::type;

template <bool VEC>
__device__ __forceinline__ Elem<VEC> load_e(const float* p, int64_t i) {
  if constexpr (VEC) {
    return ld_nt(reinterpret_cast<const float4*>(p) + i);
  } else {
    return p[i];
  }
}

template <bool VEC>
__device__ __forceinline__ void store_e(float* p, int64_t i, Elem<VEC> v) {
  if constexpr (VEC) {
    st_nt(v, reinterpret_cast<float4*>(p) + i);
  } else {
    p[i] = v;
  }
}

template <bool VEC>
__device__ __forceinline__ Elem<VEC> zero_e() {
  if constexpr (VEC) {
    return make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  } else {
    return 0.0f;
  }
}

// Push `part` into register slots holding `pushed` partials: carry through
// the occupied levels 0 .. t-1 (t = trailing ones of pushed), store at t.
template <bool VEC>
__device__ __forceinline__ void push_regs(Elem<VEC> (&st)[kLevels], int pushed, Elem<VEC> part) {
  const int t = __builtin_ctz(~pushed);
#pragma unroll
  for (int L = 0; L < kLevels; ++L)
    if (L < t) part = add_v(st[L], part);
#pragma unroll
  for (int L = 0; L < kLevels; ++L)
    if (L == t) st[L] = part;
}

// Elements [first, count) (16-byte vectors when VEC).
template <bool VEC>
__global__ __launch_bounds__(kStreamLanes) void k_replay(ReplayPtrs a, int dp_replicate, int dp_shard, int accum,
                                                float r_accum, float r_shard, float r_rep, float* out,
                                                int64_t first, int64_t count) {
  const int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  Elem<VEC> st[kLevels];
#pragma unroll
  for (int L = 0; L < kLevels; ++L) st[L] = zero_e<VEC>();
  int b = 0;
  for (int rep = 0; rep < dp_replicate; ++rep) {
    Elem<VEC> inner = zero_e<VEC>();
    for (int shard = 0; shard < dp_shard; ++shard) {
      Elem<VEC> g = zero_e<VEC>();
#pragma unroll 4
      for (int k = 0; k < accum; ++k) g = add_v(g, mul_vs(load_e<VEC>(a.p[b + k], i), r_accum));
      b += accum;
      inner = shard == 0 ? g : add_v(inner, g);
    }
    push_regs<VEC>(st, rep, mul_vs(inner, r_shard));
  }
  // Result: the lowest occupied level, then the others in ascending order.
  const int lo = __builtin_ctz(dp_replicate);
  Elem<VEC> acc = zero_e<VEC>();
#pragma unroll
  for (int L = 0; L < kLevels; ++L)
    if (L == lo) acc = st[L];
#pragma unroll
  for (int L = 0; L < kLevels; ++L)
    if (L > lo && ((dp_replicate >> L) & 1)) acc = add_v(acc, st[L]);
  store_e<VEC>(out, i, mul_vs(acc, r_rep));
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_fold_push(FoldSlotPtrs sl, int t, const float* part,
                                                   int64_t first, int64_t count) {
  const int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  Elem<VEC> carry = load_e<VEC>(part, i);
  for (int L = 0; L < t; ++L) carry = add_v(load_e<VEC>(sl.p[L], i), carry);
  store_e<VEC>(sl.p[t], i, carry);
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_fold_result(FoldSlotPtrs sl, int pushed, int average, float r,
                                                     float* __restrict__ out, int64_t first, int64_t count) {
  const int64_t i = first + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const int lo = __builtin_ctz(pushed);
  Elem<VEC> acc = load_e<VEC>(sl.p[lo], i);
  for (int L = lo + 1; L < kLevels; ++L)
    if ((pushed >> L) & 1) acc = add_v(acc, load_e<VEC>(sl.p[L], i));
  if (average) acc = mul_vs(acc, r);
  store_e<VEC>(out, i, acc);
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

unsigned grid_of(int64_t items) { return (unsigned)((items + 255) / 256); }

}  // namespace

hipError_t launch_replay(const ReplayPtrs& a, int nbuf, int dp_replicate, int dp_shard, int accum, float r_accum,
                         float r_shard, float r_rep, int64_t n, float* out, hipStream_t stream) {
  bool vec = al16(out);
  for (int b = 0; b < nbuf; ++b) vec = vec && al16(a.p[b]);
  const int64_t n4 = vec ? n / 4 : 0;
  if (n4 > 0) {
    if ((n4 + kStreamLanes - 1) / kStreamLanes > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_replay<true>, dim3((unsigned)((n4 + kStreamLanes - 1) / kStreamLanes)), dim3(kStreamLanes), 0,
                       stream, a, dp_replicate, dp_shard, accum,
                       r_accum, r_shard, r_rep, out, int64_t(0), n4);
  }
  if (4 * n4 < n) {
    const int64_t first = 4 * n4;
    if ((n - first + kStreamLanes - 1) / kStreamLanes > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_replay<false>, dim3((unsigned)((n - first + kStreamLanes - 1) / kStreamLanes)),
                       dim3(kStreamLanes), 0, stream, a, dp_replicate, dp_shard,
                       accum, r_accum, r_shard, r_rep, out, first, n);
  }
  return hipGetLastError();
}

hipError_t launch_fold_push(const FoldSlotPtrs& sl, int t, const float* part, int64_t n, hipStream_t stream) {
  bool vec = al16(part);
  for (int L = 0; L <= t; ++L) vec = vec && al16(sl.p[L]);
  const int64_t n4 = vec ? n / 4 : 0;
  if (n4 > 0)
    hipLaunchKernelGGL(k_fold_push<true>, dim3(grid_of(n4)), dim3(256), 0, stream, sl, t, part, int64_t(0), n4);
  if (4 * n4 < n)
    hipLaunchKernelGGL(k_fold_push<false>, dim3(grid_of(n - 4 * n4)), dim3(256), 0, stream, sl, t, part, 4 * n4,
                       n);
  return hipGetLastError();
}

hipError_t launch_fold_result(const FoldSlotPtrs& sl, int pushed, int average, float r, float* out, int64_t n,
                              hipStream_t stream) {
  bool vec = al16(out);
  for (int L = 0; L < kLevels; ++L)
    if ((pushed >> L) & 1) vec = vec && al16(sl.p[L]);
  const int64_t n4 = vec ? n / 4 : 0;
  if (n4 > 0)
    hipLaunchKernelGGL(k_fold_result<true>, dim3(grid_of(n4)), dim3(256), 0, stream, sl, pushed, average, r, out,
                       int64_t(0), n4);
  if (4 * n4 < n)
    hipLaunchKernelGGL(k_fold_result<false>, dim3(grid_of(n - 4 * n4)), dim3(256), 0, stream, sl, pushed, average,
                       r, out, 4 * n4, n);
  return hipGetLastError();
}

}  // namespace repro
