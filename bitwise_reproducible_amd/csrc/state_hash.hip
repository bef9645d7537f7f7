// repro_state_hash: BLAKE2b tree digest of the flat binary32 state.
//
// "OPEN-1B: A Fully Auditable Training Run", Appendix B (a canonical state
// hash anchors every step) and the legend of Figure 11 (the hash is
// BLAKE2b); section 3.2 (optimizer state hashed in FP32).  The function is
// BLAKE2b of RFC 7693 in the tree mode of the BLAKE2 paper (section 2.10):
// digest 32 bytes, fanout 16, depth 255, leaf length 4096, inner length 32,
// personalisation "repro_state_v1"; see repro.h for the full tree shape.
//
// Design for gfx950: hashing is integer-ALU bound (each 128-byte block costs
// 12 rounds x 8 G-functions of 64-bit add/xor/rotate, i.e. roughly 20 32-bit
// VALU operations per byte), so the kernels aim at full VALU occupancy
// rather than at HBM bandwidth:
//  - one lane per 4 KiB leaf (32 compressions), all rounds unrolled so the
//    message schedule is resolved at compile time and the 16 message words,
//    the 16 state words and the chaining value stay in VGPRs;
//  - each block's eight 16-byte loads are issued right before it is
//    compressed; at 100 VGPRs four waves share a SIMD and hide the load
//    latency (prefetching the next block instead costs 32 more VGPRs, one
//    wave fewer, and measured 2% slower);
//  - upper levels with many nodes run one lane per node (a node reads 16
//    digests = 512 bytes = 4 compressions); the last levels (at most
//    kTailNodes nodes) run in one workgroup with a barrier between levels,
//    which also writes the root digest.
#include <hip/hip_runtime.h>

#include "device_ops.h"
#include "internal.h"

namespace repro {
namespace {

constexpr int kLeafBytes = 4096;
constexpr int kFanout = 16;
constexpr int kDigest = 32;
constexpr int kTailNodes = 256;

__constant__ uint64_t kIV[8] = {0x6A09E667F3BCC908ULL, 0xBB67AE8584CAA73BULL, 0x3C6EF372FE94F82BULL,
                                0xA54FF53A5F1D36F1ULL, 0x510E527FADE682D1ULL, 0x9B05688C2B3E6C1FULL,
                                0x1F83D9ABFB41BD6BULL, 0x5BE0CD19137E2179ULL};

// RFC 7693 message schedule; rounds 10 and 11 reuse rows 0 and 1.
constexpr uint8_t kSigma[12][16] = {
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15}, {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3},
    {11, 8, 12, 0, 5, 2, 15, 13, 10, 14, 3, 6, 7, 1, 9, 4}, {7, 9, 3, 1, 13, 12, 11, 14, 2, 6, 5, 10, 4, 0, 15, 8},
    {9, 0, 5, 7, 2, 4, 10, 15, 14, 1, 11, 12, 6, 8, 3, 13}, {2, 12, 6, 10, 0, 11, 8, 3, 4, 13, 7, 5, 15, 14, 1, 9},
    {12, 5, 1, 15, 14, 13, 4, 10, 0, 7, 6, 3, 9, 2, 8, 11}, {13, 11, 7, 14, 12, 1, 3, 9, 5, 0, 15, 4, 8, 6, 2, 10},
    {6, 15, 14, 9, 11, 3, 0, 8, 12, 2, 13, 7, 1, 4, 10, 5}, {10, 2, 8, 4, 7, 6, 1, 5, 15, 11, 9, 14, 3, 12, 13, 0},
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15}, {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3}};

// Parameter-block words 0, 2, 6, 7 (word 1 is the node offset, words 3-5
// are reserved or salt and zero):
//   word 0: digest 32 | key 0 | fanout 16 | depth 255 | leaf length 4096
//   word 2: node depth | inner length 32 << 8
//   words 6, 7: "repro_st", "ate_v1\0\0" little-endian
constexpr uint64_t kParam0 = 0x20ULL | (0x00ULL << 8) | (0x10ULL << 16) | (0xFFULL << 24) |
                             ((uint64_t)kLeafBytes << 32);
constexpr uint64_t kPersonal0 = 0x74735F6F72706572ULL;
constexpr uint64_t kPersonal1 = 0x000031765F657461ULL;

// Rotation right by R of a 64-bit word held as two 32-bit halves.  By 32 it
// is a swap of the halves (no instruction); by 24, 16 and 63 it is two
// v_alignbit_b32 (each takes a 64-bit pair and returns one 32-bit window),
// which measured 11% faster over the whole hash than the compiler's 64-bit
// shift-and-or sequences (about three instructions per rotation).
template <int R>
__device__ __forceinline__ uint64_t rotr(uint64_t x) {
  if constexpr (R == 32) {
    return (x >> 32) | (x << 32);
  } else {
    constexpr int n = R < 32 ? R : R - 32;
    const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
    const uint32_t a = R < 32 ? hi : lo;  // by R >= 32: swap the halves, then rotate by R - 32
    const uint32_t b = R < 32 ? lo : hi;
    const uint32_t nlo = __builtin_amdgcn_alignbit(a, b, n);
    const uint32_t nhi = __builtin_amdgcn_alignbit(b, a, n);
    return ((uint64_t)nhi << 32) | nlo;
  }
}

template <int A, int B, int C, int D>
__device__ __forceinline__ void g_mix(uint64_t (&v)[16], uint64_t x, uint64_t y) {
  v[A] = v[A] + v[B] + x;
  v[D] = rotr<32>(v[D] ^ v[A]);
  v[C] = v[C] + v[D];
  v[B] = rotr<24>(v[B] ^ v[C]);
  v[A] = v[A] + v[B] + y;
  v[D] = rotr<16>(v[D] ^ v[A]);
  v[C] = v[C] + v[D];
  v[B] = rotr<63>(v[B] ^ v[C]);
}

template <int RND>
__device__ __forceinline__ void round_fn(uint64_t (&v)[16], const uint64_t (&m)[16]) {
  constexpr const uint8_t* s = kSigma[RND];
  g_mix<0, 4, 8, 12>(v, m[s[0]], m[s[1]]);
  g_mix<1, 5, 9, 13>(v, m[s[2]], m[s[3]]);
  g_mix<2, 6, 10, 14>(v, m[s[4]], m[s[5]]);
  g_mix<3, 7, 11, 15>(v, m[s[6]], m[s[7]]);
  g_mix<0, 5, 10, 15>(v, m[s[8]], m[s[9]]);
  g_mix<1, 6, 11, 12>(v, m[s[10]], m[s[11]]);
  g_mix<2, 7, 8, 13>(v, m[s[12]], m[s[13]]);
  g_mix<3, 4, 9, 14>(v, m[s[14]], m[s[15]]);
}

template <int RND>
__device__ __forceinline__ void rounds_from(uint64_t (&v)[16], const uint64_t (&m)[16]) {
  if constexpr (RND < 12) {
    round_fn<RND>(v, m);
    rounds_from<RND + 1>(v, m);
  }
}

// Compression F(h, m, t, f): `t` is the byte count including this block
// (below 2^64 here, so the high counter word is zero).
__device__ __forceinline__ void compress(uint64_t (&h)[8], const uint64_t (&m)[16], uint64_t t, bool last_block,
                                         bool last_node) {
  uint64_t v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = h[i];
    v[i + 8] = kIV[i];
  }
  v[12] ^= t;
  if (last_block) v[14] = ~v[14];
  if (last_block && last_node) v[15] = ~v[15];
  rounds_from<0>(v, m);
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] ^= v[i] ^ v[i + 8];
}

__device__ __forceinline__ void init_node(uint64_t (&h)[8], uint64_t node_offset, int node_depth) {
  h[0] = kIV[0] ^ kParam0;
  h[1] = kIV[1] ^ node_offset;
  h[2] = kIV[2] ^ ((uint64_t)node_depth | ((uint64_t)kDigest << 8));
  h[3] = kIV[3];
  h[4] = kIV[4];
  h[5] = kIV[5];
  h[6] = kIV[6] ^ kPersonal0;
  h[7] = kIV[7] ^ kPersonal1;
}

__device__ __forceinline__ void load_block16(uint64_t (&m)[16], const uint4* __restrict__ p) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 u = p[q];
    m[2 * q] = (uint64_t)u.x | ((uint64_t)u.y << 32);
    m[2 * q + 1] = (uint64_t)u.z | ((uint64_t)u.w << 32);
  }
}

__device__ __forceinline__ void store_digest(uint8_t* __restrict__ out, const uint64_t (&h)[8]) {
  uint4* o = reinterpret_cast<uint4*>(out);
  o[0] = make_uint4((uint32_t)h[0], (uint32_t)(h[0] >> 32), (uint32_t)h[1], (uint32_t)(h[1] >> 32));
  o[1] = make_uint4((uint32_t)h[2], (uint32_t)(h[2] >> 32), (uint32_t)h[3], (uint32_t)(h[3] >> 32));
}

// Hash `len` bytes of 32-bit words at `w` (len a multiple of 4), reading
// word by word with zero padding; used for a short last leaf and for
// unaligned inputs.
__device__ void hash_words_generic(uint64_t (&h)[8], const uint32_t* __restrict__ w, uint64_t len,
                                   bool last_node) {
  const uint64_t nblocks = len == 0 ? 1 : (len + 127) / 128;
  for (uint64_t b = 0; b < nblocks; ++b) {
    uint64_t m[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint64_t byte = b * 128 + 8 * q;
      const uint32_t lo = byte < len ? w[byte / 4] : 0u;
      const uint32_t hi = byte + 4 < len ? w[byte / 4 + 1] : 0u;
      m[q] = (uint64_t)lo | ((uint64_t)hi << 32);
    }
    const bool last = b + 1 == nblocks;
    const uint64_t t = last ? len : (b + 1) * 128;
    compress(h, m, t, last, last_node);
  }
}

// Level 0.  One lane per leaf.  Full leaves of a 16-byte aligned input take
// the pipelined path; the last leaf, if short, and unaligned inputs take the
// word-by-word path.
// The leaves of `ranges` equal runs of `count` leaves starting at
// first + r * stride (r = 0 .. ranges-1), of `leaves` in all: one run for a
// whole level, or the same span of w, m and v after an update chunk.
template <bool ALIGNED>
__global__ __launch_bounds__(256) void k_hash_leaves(const float* __restrict__ words, uint64_t nbytes,
                                                      int64_t leaves, int64_t first, int64_t count, int64_t stride,
                                                      int ranges, uint8_t* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= count * ranges) return;
  const int64_t r = k / count;
  const int64_t i = first + r * stride + (k - r * count);
  uint64_t h[8];
  init_node(h, (uint64_t)i, 0);
  const bool last_node = i == leaves - 1;
  const uint64_t start = (uint64_t)i * kLeafBytes;
  const uint64_t len = nbytes - start < (uint64_t)kLeafBytes ? nbytes - start : (uint64_t)kLeafBytes;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(words) + start / 4;
  if (ALIGNED && len == (uint64_t)kLeafBytes) {
    const uint4* p = reinterpret_cast<const uint4*>(w);
    for (int b = 0; b < kLeafBytes / 128; ++b) {
      uint64_t m[16];
      load_block16(m, p + 8 * b);
      const bool last = b + 1 == kLeafBytes / 128;
      compress(h, m, (uint64_t)(b + 1) * 128, last, last_node);
    }
  } else {
    hash_words_generic(h, w, len, last_node);
  }
  store_digest(out + 32 * i, h);
}

// Hash one inner node: children [c0, c0 + nc) of the level below.
__device__ __forceinline__ void hash_inner(uint64_t (&h)[8], const uint8_t* __restrict__ below, int64_t c0,
                                           int nc, bool last_node) {
  // nc digests of 32 bytes = nc/4 full blocks (nc <= 16), zero padded.
  const uint4* p = reinterpret_cast<const uint4*>(below + 32 * c0);
  const int len = nc * kDigest;
  const int nblocks = (len + 127) / 128;
  for (int b = 0; b < nblocks; ++b) {
    uint64_t m[16];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int byte = b * 128 + 16 * q;
      const uint4 u = byte < len ? p[byte / 16] : make_uint4(0, 0, 0, 0);
      m[2 * q] = (uint64_t)u.x | ((uint64_t)u.y << 32);
      m[2 * q + 1] = (uint64_t)u.z | ((uint64_t)u.w << 32);
    }
    const bool last = b + 1 == nblocks;
    compress(h, m, last ? (uint64_t)len : (uint64_t)(b + 1) * 128, last, last_node);
  }
}

__global__ __launch_bounds__(256) void k_hash_level(const uint8_t* __restrict__ below, int64_t count_below,
                                                     uint8_t* __restrict__ out, int64_t count, int depth) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= count) return;
  const int64_t c0 = j * kFanout;
  const int nc = (int)(count_below - c0 < kFanout ? count_below - c0 : kFanout);
  uint64_t h[8];
  init_node(h, (uint64_t)j, depth);
  hash_inner(h, below, c0, nc, j == count - 1);
  store_digest(out + 32 * j, h);
}

struct TailPlan {
  int first_level;  // first level this kernel computes (>= 1)
  int levels;       // total levels, leaves included
  int64_t count[HashPlan::kMaxLevels];
  int64_t offset[HashPlan::kMaxLevels];
};

// The last levels, each with at most kTailNodes nodes, in one workgroup.
__global__ __launch_bounds__(kTailNodes) void k_hash_tail(uint8_t* __restrict__ ws, TailPlan plan,
                                                           uint8_t* __restrict__ digest_out) {
  for (int d = plan.first_level; d < plan.levels; ++d) {
    const int64_t count = plan.count[d];
    const int64_t below_count = plan.count[d - 1];
    for (int64_t j = threadIdx.x; j < count; j += blockDim.x) {
      const int64_t c0 = j * kFanout;
      const int nc = (int)(below_count - c0 < kFanout ? below_count - c0 : kFanout);
      uint64_t h[8];
      init_node(h, (uint64_t)j, d);
      hash_inner(h, ws + plan.offset[d - 1], c0, nc, j == count - 1);
      store_digest(ws + plan.offset[d] + 32 * j, h);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const uint4* root = reinterpret_cast<const uint4*>(ws + plan.offset[plan.levels - 1]);
    uint4* o = reinterpret_cast<uint4*>(digest_out);
    o[0] = root[0];
    o[1] = root[1];
  }
}

// ---------------------------------------------------------------------------
// AdamW and the leaf level of the state hash in one pass (n a multiple of
// 1024, so every 4 KiB leaf lies inside one of w, m and v).
//
// A workgroup is one wave; it owns kTriples = 21 leaf indices j and so the
// 63 leaves w_j, m_j, v_j (leaf numbers j, n/1024 + j, 2n/1024 + j), one per
// lane (lane 63 only helps with the update).  For each of the 32 blocks b of
// a leaf, the wave updates elements 1024 j + 32 b .. + 31 of every owned j
// (whole 128-byte runs of w, m, v, g), stores w', m', v' to HBM and the same
// bytes to LDS, and then each lane compresses block b of its leaf from LDS.
// The barriers between the two phases involve this wave alone, so waves
// never wait for one another; the updated state is never read back.
constexpr int kTriples = 21;
constexpr int kFusedThreads = 64;

__global__ __launch_bounds__(kFusedThreads) void k_adamw_hash_leaves(float* __restrict__ state,
                                                                     const float* __restrict__ grad, int64_t n,
                                                                     AdamwScalars s, uint8_t* __restrict__ out) {
  // One 128-byte block per leaf, rows padded to 144 bytes so that 16 lanes
  // reading 16 bytes at a time from consecutive rows hit 64 distinct banks.
  __shared__ uint4 rows[3 * kTriples][9];
  const int tid = threadIdx.x;
  const int64_t per_region = n / 1024;
  const int64_t j0 = (int64_t)blockIdx.x * kTriples;
  const int T = per_region - j0 < kTriples ? (int)(per_region - j0) : kTriples;
  const int region = tid / kTriples;
  const int q = tid - region * kTriples;
  const bool hashing = tid < 3 * kTriples && q < T;
  const int64_t leaf = region * per_region + j0 + q;
  const bool last_node = leaf == 3 * per_region - 1;
  uint64_t h[8];
  init_node(h, (uint64_t)leaf, 0);
  float4* W = reinterpret_cast<float4*>(state);
  float4* M = reinterpret_cast<float4*>(state + n);
  float4* V = reinterpret_cast<float4*>(state + 2 * n);
  const float4* G = reinterpret_cast<const float4*>(grad);
  for (int b = 0; b < kLeafBytes / 128; ++b) {
    for (int f = tid; f < 8 * T; f += kFusedThreads) {
      const int qq = f >> 3;
      const int e4 = f & 7;
      const int64_t i4 = (j0 + qq) * 256 + 8 * b + e4;  // element (j0 + qq) * 1024 + 32 b + 4 e4
      float4 w = ld_nt(W + i4);
      float4 m = ld_nt(M + i4);
      float4 v = ld_nt(V + i4);
      const float4 g = ld_nt(G + i4);
      adamw_elem(w.x, m.x, v.x, g.x, s);
      adamw_elem(w.y, m.y, v.y, g.y, s);
      adamw_elem(w.z, m.z, v.z, g.z, s);
      adamw_elem(w.w, m.w, v.w, g.w, s);
      st_nt(w, W + i4);
      st_nt(m, M + i4);
      st_nt(v, V + i4);
      rows[qq][e4] = make_uint4(__float_as_uint(w.x), __float_as_uint(w.y), __float_as_uint(w.z),
                                __float_as_uint(w.w));
      rows[kTriples + qq][e4] = make_uint4(__float_as_uint(m.x), __float_as_uint(m.y), __float_as_uint(m.z),
                                           __float_as_uint(m.w));
      rows[2 * kTriples + qq][e4] = make_uint4(__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                               __float_as_uint(v.w));
    }
    __syncthreads();
    if (hashing) {
      uint64_t mw[16];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint4 u = rows[tid][k];
        mw[2 * k] = (uint64_t)u.x | ((uint64_t)u.y << 32);
        mw[2 * k + 1] = (uint64_t)u.z | ((uint64_t)u.w << 32);
      }
      const bool last = b + 1 == kLeafBytes / 128;
      compress(h, mw, (uint64_t)(b + 1) * 128, last, last_node);
    }
    __syncthreads();
  }
  if (hashing) store_digest(out + 32 * leaf, h);
}

}  // namespace

hipError_t launch_adamw_hash_fused(float* state, const float* grad, int64_t n, const AdamwScalars& s, uint8_t* ws,
                                   const HashPlan& plan, uint8_t* digest_out, hipStream_t stream) {
  if (n <= 0 || n % 1024 != 0) return hipErrorInvalidValue;
  const int64_t grid = (n / 1024 + kTriples - 1) / kTriples;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_adamw_hash_leaves, dim3((unsigned)grid), dim3(kFusedThreads), 0, stream, state, grad, n, s,
                     ws + plan.offset[0]);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_hash_upper(ws, plan, digest_out, stream);
}

void plan_state_hash(int64_t n_words, HashPlan* plan) {
  const uint64_t nbytes = (uint64_t)n_words * 4u;
  int64_t count = nbytes == 0 ? 1 : (int64_t)((nbytes + kLeafBytes - 1) / kLeafBytes);
  int levels = 0;
  int64_t offset = 0;
  for (;;) {
    plan->count[levels] = count;
    plan->offset[levels] = offset;
    offset += ((count * kDigest + 255) / 256) * 256;
    ++levels;
    if (count == 1 && levels >= 2) break;
    count = (count + kFanout - 1) / kFanout;
  }
  plan->levels = levels;
  plan->total_bytes = offset;
}

hipError_t launch_hash_leaves(const float* words, int64_t n_words, uint8_t* ws, const HashPlan& plan, int64_t first,
                              int64_t count, int64_t stride, int ranges, hipStream_t stream) {
  const uint64_t nbytes = (uint64_t)n_words * 4u;
  const int64_t leaves = plan.count[0];
  if (first < 0 || count < 0 || stride < 0 || ranges < 1 || first + (ranges - 1) * stride + count > leaves)
    return hipErrorInvalidValue;
  if (count == 0) return hipSuccess;
  const bool aligned = (reinterpret_cast<uintptr_t>(words) & 15u) == 0;
  const int64_t grid0 = (count * ranges + 255) / 256;
  if (grid0 > 0x7fffffff) return hipErrorInvalidValue;
  if (aligned)
    hipLaunchKernelGGL(k_hash_leaves<true>, dim3((unsigned)grid0), dim3(256), 0, stream, words, nbytes, leaves,
                       first, count, stride, ranges, ws + plan.offset[0]);
  else
    hipLaunchKernelGGL(k_hash_leaves<false>, dim3((unsigned)grid0), dim3(256), 0, stream, words, nbytes, leaves,
                       first, count, stride, ranges, ws + plan.offset[0]);
  return hipGetLastError();
}

hipError_t launch_state_hash(const float* words, int64_t n_words, uint8_t* ws, const HashPlan& plan,
                             uint8_t* digest_out, hipStream_t stream) {
  const hipError_t e = launch_hash_leaves(words, n_words, ws, plan, 0, plan.count[0], 0, 1, stream);
  if (e != hipSuccess) return e;
  return launch_hash_upper(ws, plan, digest_out, stream);
}

hipError_t launch_hash_upper(uint8_t* ws, const HashPlan& plan, uint8_t* digest_out, hipStream_t stream) {
  int d = 1;
  for (; d < plan.levels && plan.count[d] > kTailNodes; ++d) {
    const int64_t grid = (plan.count[d] + 255) / 256;
    hipLaunchKernelGGL(k_hash_level, dim3((unsigned)grid), dim3(256), 0, stream, ws + plan.offset[d - 1],
                       plan.count[d - 1], ws + plan.offset[d], plan.count[d], d);
  }
  TailPlan tp;
  tp.first_level = d;
  tp.levels = plan.levels;
  for (int i = 0; i < plan.levels; ++i) {
    tp.count[i] = plan.count[i];
    tp.offset[i] = plan.offset[i];
  }
  hipLaunchKernelGGL(k_hash_tail, dim3(1), dim3(kTailNodes), 0, stream, ws, tp, digest_out);
  return hipGetLastError();
}

}  // namespace repro
