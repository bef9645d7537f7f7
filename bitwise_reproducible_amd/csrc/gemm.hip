// repro_gemm: C = op(A) * op(B) with one ascending-k chain per output.
//
// "OPEN-1B: A Fully Auditable Training Run", section 2.1 ("Reduction order":
// every sum inside a matrix multiply in one fixed order; "Fused
// multiply-add": explicitly unfused multiply and add on the GPU) and section
// 6, item 1.  The declared order: acc = +0, then for k = 0, 1, ..., K-1,
// acc = fl(acc + fl(a_ik * b_kj)).
//
// Design for gfx950:
//  - gfx950 has no unfused multiply-add instruction, and fused ones round
//    once, so every step is a rounded product and a v_add_f32.  The default
//    kernel (k_gemm_mfma) forms the products on the matrix cores:
//    v_mfma_f32_32x32x1_2b_f32 with K = 1 and C = -0 returns fl(a * b) for
//    2,048 pairs at once.  The VALU kernel (k_gemm) uses v_mul_f32.  The
//    matrix cores and the VALU take turns on a SIMD and the products cost
//    the same SIMD time either way; the matrix-core form holds a higher
//    clock.  The file is built with -ffp-contract=off and without
//    packed-fp32 instructions; the instruction-mix audit in the tests checks
//    that no v_fma / v_fmac / v_pk_* appears in the unfused kernels.
//  - repro_gemm_fma declares the other convention (one fused step per k);
//    its kernels, k_gemm_fma (v_fma_f32) and k_gemm_mfma_fma (matrix cores),
//    share the tiling below and differ only in the step.
//  - It is built with -fgpu-flush-denormals-to-zero: the kernel descriptor
//    sets the fp32 denormal mode to "flush inputs and outputs", so the VALU
//    itself applies the subnormal rule of section 2.1 at no cost (on gfx950
//    this flush is the x86 FTZ/DAZ rule bit for bit; repro_fp32_ops exposes
//    the same v_mul_f32 / v_add_f32 for the directed boundary tests).
//  - Work is split over output tiles only.  A workgroup of 256 lanes owns a
//    BM x BN tile and walks the K dimension in ascending BK-wide slabs
//    staged through LDS (double buffered, one barrier per slab); each lane
//    (VALU kernel: a TM x TN register tile) or each wave (matrix cores: a
//    64 x 64 tile held in the instructions' output registers) keeps every
//    output's single serial chain in its own register.  No split-k, no
//    atomics, no cross-lane sums.
//  - A and B slabs are loaded with 16-byte global loads when the layout
//    allows and stored k-major in LDS, so that the inner loop reads a and b
//    fragments (VALU: 16-byte vectors) or matrix operands (one word per
//    lane) with few bank conflicts.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.h"

namespace repro {
namespace {

template <int BM, int BN, int BK, int TM, int TN, bool TA, bool TB, bool VEC>
struct GemmTile {
  static constexpr int TX = BN / TN;  // lanes along n
  static constexpr int TY = BM / TM;  // lanes along m
  static constexpr int NT = TX * TY;  // lanes per workgroup
  static_assert(TM % 4 == 0 && TN % 4 == 0, "register tiles are read as 16-byte vectors");
};

// Loads one slab chunk (4 consecutive elements along the contiguous
// dimension of the stored matrix) with bounds checks; out-of-range elements
// read as zero and are never used by an in-range output.
template <bool VEC>
__device__ __forceinline__ float4 load_chunk(const float* __restrict__ p, int64_t row, int64_t col, int64_t ld,
                                             int64_t rows, int64_t cols) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row < rows) {
    const float* q = p + row * ld + col;
    if constexpr (VEC) {
      if (col < cols) v = *reinterpret_cast<const float4*>(q);
    } else {
      if (col + 0 < cols) v.x = q[0];
      if (col + 1 < cols) v.y = q[1];
      if (col + 2 < cols) v.z = q[2];
      if (col + 3 < cols) v.w = q[3];
    }
  }
  return v;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Byte offsets inside one slab fit in 32 bits for these leading dimensions
// (every lane's offset from the slab's base below 2^32 bytes).
template <int BM, int BN, int BK, bool TA, bool TB>
bool slab_offsets_fit(int64_t lda, int64_t ldb) {
  const int64_t a_span = TA ? (int64_t)BK * lda + BM : (int64_t)BM * lda + BK;
  const int64_t b_span = TB ? (int64_t)BN * ldb + BK : (int64_t)BK * ldb + BN;
  return lda < ((int64_t)1 << 40) && ldb < ((int64_t)1 << 40) && 4 * a_span < ((int64_t)1 << 32) &&
         4 * b_span < ((int64_t)1 << 32);
}

// Staging of the BK-deep k slabs of op(A) (BM rows) and op(B) (BN columns)
// for a workgroup of NT lanes: global memory -> registers -> LDS, k-major in
// LDS (double-buffered), shared by the VALU and matrix-core tiles.  Each
// lane loads 16-byte chunks along the stored matrix's contiguous dimension.
// LDS rows are padded by APAD / BPAD floats: 4 keeps rows 16-byte aligned
// (the VALU tiles read 16-byte fragments, and untransposed slabs are stored
// 16 bytes at a time); the matrix-core tiles read single words and take 2
// for a slab that is transposed on its way into LDS.
template <int BM, int BN, int BK, int NT, bool TA, bool TB, bool VEC, int APAD = 4, int BPAD = 4>
struct SlabStager {
  static constexpr int LA = BM * BK / 4 / NT;  // 4-element chunks of A per lane per slab
  static constexpr int LB = BK * BN / 4 / NT;
  static_assert(LA * NT * 4 == BM * BK && LB * NT * 4 == BK * BN, "slab must split evenly over lanes");
  static_assert(BK % 4 == 0, "BK must be a multiple of 4");
  static_assert((!TA || APAD % 4 == 0) && (TB || BPAD % 4 == 0),
                "slabs stored 16 bytes at a time need 16-byte aligned rows");
  typedef float ASlab[BK][BM + APAD];
  typedef float BSlab[BK][BN + BPAD];

  ASlab* As;  // [2], in LDS
  BSlab* Bs;
  const float* A;
  const float* B;
  int64_t lda, ldb, M, N, K, i0, j0;
  int tid;
  // Interior tiles: a wave-uniform slab base and per-lane 32-bit offsets.
  const char* abase;
  const char* bbase;
  int64_t astep, bstep;
  uint32_t oa[LA], ob[LB];
  v4f ra[LA], rb[LB];

  __device__ __forceinline__ SlabStager(ASlab* As_, BSlab* Bs_, const float* A_, int64_t lda_, const float* B_,
                                        int64_t ldb_, int64_t M_, int64_t N_, int64_t K_, int64_t i0_,
                                        int64_t j0_, int tid_)
      : As(As_), Bs(Bs_), A(A_), B(B_), lda(lda_), ldb(ldb_), M(M_), N(N_), K(K_), i0(i0_), j0(j0_), tid(tid_) {
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int f = tid + q * NT;
      oa[q] = !TA ? (uint32_t)(4 * ((int64_t)(f / (BK / 4)) * lda + 4 * (f % (BK / 4))))
                  : (uint32_t)(4 * ((int64_t)(f / (BM / 4)) * lda + 4 * (f % (BM / 4))));
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int f = tid + q * NT;
      ob[q] = !TB ? (uint32_t)(4 * ((int64_t)(f / (BN / 4)) * ldb + 4 * (f % (BN / 4))))
                  : (uint32_t)(4 * ((int64_t)(f / (BK / 4)) * ldb + 4 * (f % (BK / 4))));
    }
    abase = reinterpret_cast<const char*>(TA ? A + i0 : A + i0 * lda);
    bbase = reinterpret_cast<const char*>(TB ? B + j0 * ldb : B + j0);
    astep = 4 * (TA ? BK * lda : BK);
    bstep = 4 * (TB ? BK : BK * ldb);
  }

  // Global -> registers for the slab starting at k0, bounds-checked.
  __device__ __forceinline__ void load_checked(int64_t k0) {
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int f = tid + q * NT;
      float4 v;
      if constexpr (!TA) {  // A is M x K row-major: rows i, contiguous k
        const int r = f / (BK / 4), c4 = f % (BK / 4);
        v = load_chunk<VEC>(A, i0 + r, k0 + 4 * c4, lda, M, K);
      } else {  // A stored K x M: rows k, contiguous i
        const int c = f / (BM / 4), r4 = f % (BM / 4);
        v = load_chunk<VEC>(A, k0 + c, i0 + 4 * r4, lda, K, M);
      }
      ra[q] = v4f{v.x, v.y, v.z, v.w};
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int f = tid + q * NT;
      float4 v;
      if constexpr (!TB) {  // B is K x N row-major: rows k, contiguous j
        const int c = f / (BN / 4), j4 = f % (BN / 4);
        v = load_chunk<VEC>(B, k0 + c, j0 + 4 * j4, ldb, K, N);
      } else {  // B stored N x K: rows j, contiguous k
        const int j = f / (BK / 4), c4 = f % (BK / 4);
        v = load_chunk<VEC>(B, j0 + j, k0 + 4 * c4, ldb, N, K);
      }
      rb[q] = v4f{v.x, v.y, v.z, v.w};
    }
  }

  // Global -> registers for slab s of an interior tile: no bounds checks.
  __device__ __forceinline__ void load_interior(int64_t s) {
    const char* ab = abase + s * astep;
    const char* bb = bbase + s * bstep;
#pragma unroll
    for (int q = 0; q < LA; ++q) ra[q] = *reinterpret_cast<const v4f*>(ab + oa[q]);
#pragma unroll
    for (int q = 0; q < LB; ++q) rb[q] = *reinterpret_cast<const v4f*>(bb + ob[q]);
  }

  // Registers -> LDS buffer `buf`, k-major.
  __device__ __forceinline__ void store(int buf) {
#pragma unroll
    for (int q = 0; q < LA; ++q) {
      const int f = tid + q * NT;
      if constexpr (!TA) {
        const int r = f / (BK / 4), c4 = f % (BK / 4);
        As[buf][4 * c4 + 0][r] = ra[q].x;
        As[buf][4 * c4 + 1][r] = ra[q].y;
        As[buf][4 * c4 + 2][r] = ra[q].z;
        As[buf][4 * c4 + 3][r] = ra[q].w;
      } else {
        const int c = f / (BM / 4), r4 = f % (BM / 4);
        *reinterpret_cast<v4f*>(&As[buf][c][4 * r4]) = ra[q];
      }
    }
#pragma unroll
    for (int q = 0; q < LB; ++q) {
      const int f = tid + q * NT;
      if constexpr (!TB) {
        const int c = f / (BN / 4), j4 = f % (BN / 4);
        *reinterpret_cast<v4f*>(&Bs[buf][c][4 * j4]) = rb[q];
      } else {
        const int j = f / (BK / 4), c4 = f % (BK / 4);
        Bs[buf][4 * c4 + 0][j] = rb[q].x;
        Bs[buf][4 * c4 + 1][j] = rb[q].y;
        Bs[buf][4 * c4 + 2][j] = rb[q].z;
        Bs[buf][4 * c4 + 3][j] = rb[q].w;
      }
    }
  }
};

// The k loop of a tile: slabs 0 .. K/BK - 1 are full, a last, partial one
// holds K % BK steps; `full_slab(buf)` runs the BK steps of a staged slab in
// ascending order and `step(buf, kk)` one step.  Interior tiles (the whole
// tile inside C, 16-byte rows, 32-bit slab offsets, K a whole number of
// slabs) and the others run separate copies of the loop: the same steps in
// the same order, other loads.  The loop body is the same on every pass (a
// conditional prefetch makes the compiler spill): an interior tile reloads
// its last slab on the last pass and the bounds-checked loads read past K
// as zeros, into the buffer that is no longer read.
template <int BK, class Stager, class FullSlab, class Step>
__device__ __forceinline__ void run_k_loop(Stager& st, bool interior, int64_t K, FullSlab full_slab, Step step) {
  const int64_t nfull = K / BK;
  auto run = [&](auto interior_tag) __attribute__((always_inline)) {
    constexpr bool kInterior = decltype(interior_tag)::value;
    if constexpr (kInterior) {
      st.load_interior(0);
    } else {
      st.load_checked(0);
    }
    st.store(0);
    __syncthreads();
    int buf = 0;
    for (int64_t s = 0; s < nfull; ++s) {
      if constexpr (kInterior) {
        st.load_interior(s + 1 < nfull ? s + 1 : s);
      } else {
        st.load_checked((s + 1) * BK);
      }
      full_slab(buf);
      st.store(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    if constexpr (!kInterior) {
      const int kleft = (int)(K - nfull * BK);
      for (int kk = 0; kk < kleft; ++kk) step(buf, kk);
    }
  };
  if (interior && K % BK == 0 && nfull > 0) {
    run(std::true_type{});
  } else if (K > 0) {
    run(std::false_type{});
  }
}

template <int BM, int BN, int BK, int TM, int TN, bool TA, bool TB, bool VEC, bool FUSED>
__device__ __forceinline__ void gemm_tile(int64_t M, int64_t N, int64_t K, const float* __restrict__ A,
                                          int64_t lda, const float* __restrict__ B, int64_t ldb,
                                          float* __restrict__ C, int64_t ldc, int tiles_n, int off32) {
  using T = GemmTile<BM, BN, BK, TM, TN, TA, TB, VEC>;
  using S = SlabStager<BM, BN, BK, T::NT, TA, TB, VEC>;
  __shared__ __attribute__((aligned(16))) typename S::ASlab As[2];
  __shared__ __attribute__((aligned(16))) typename S::BSlab Bs[2];

  const int tile = blockIdx.x;
  const int64_t i0 = (int64_t)(tile / tiles_n) * BM;
  const int64_t j0 = (int64_t)(tile % tiles_n) * BN;
  const int tid = threadIdx.x;
  const int tx = tid % T::TX;
  const int ty = tid / T::TX;
  S st(As, Bs, A, lda, B, ldb, M, N, K, i0, j0, tid);

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;  // the chain starts at +0

  // Register fragments of one k step: the lane's TM values of A and TN of B.
  float fa[2][TM], fb[2][TN];
  auto read_frag = [&](int slot, int buf, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < TM / 4; ++g)
      *reinterpret_cast<v4f*>(&fa[slot][4 * g]) =
          *reinterpret_cast<const v4f*>(&As[buf][kk][g * 4 * T::TY + ty * 4]);
#pragma unroll
    for (int g = 0; g < TN / 4; ++g)
      *reinterpret_cast<v4f*>(&fb[slot][4 * g]) =
          *reinterpret_cast<const v4f*>(&Bs[buf][kk][g * 4 * T::TX + tx * 4]);
  };
  // One k step: every output of the lane takes fl(acc + fl(a * b)), or
  // fl(a * b + acc) rounded once under the fused convention.
  auto mac_frag = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if constexpr (FUSED) {
          acc[i][j] = __builtin_fmaf(fa[slot][i], fb[slot][j], acc[i][j]);
        } else {
          const float p = fa[slot][i] * fb[slot][j];
          acc[i][j] = acc[i][j] + p;
        }
      }
  };
  // A full slab, k ascending.  The LDS reads of step kk + 1 are issued
  // before the multiplies of step kk (the scheduling barriers keep the
  // compiler from sinking them to their use), so a wave does not wait on LDS
  // latency between steps; this only moves loads, never the order of a chain.
  auto full_slab = [&](int buf) __attribute__((always_inline)) {
    read_frag(0, buf, 0);
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      if (kk + 1 < BK) read_frag((kk + 1) & 1, buf, kk + 1);
      __builtin_amdgcn_sched_barrier(0);
      mac_frag(kk & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto step = [&](int buf, int kk) __attribute__((always_inline)) {
    read_frag(0, buf, kk);
    mac_frag(0);
  };
  const bool interior = VEC && off32 && i0 + BM <= M && j0 + BN <= N;
  run_k_loop<BK>(st, interior, K, full_slab, step);

  // Epilogue: lane rows g*4*TY + ty*4 + e, columns h*4*TX + tx*4 + 0..3.
  const bool vec_c = VEC && (ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15u) == 0);
#pragma unroll
  for (int g = 0; g < TM / 4; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = i0 + g * 4 * T::TY + ty * 4 + e;
      if (row >= M) continue;
#pragma unroll
      for (int h = 0; h < TN / 4; ++h) {
        const int64_t col = j0 + h * 4 * T::TX + tx * 4;
        float* out = C + row * ldc + col;
        const float* v = &acc[g * 4 + e][h * 4];
        if (vec_c && col + 3 < N) {
          *reinterpret_cast<float4*>(out) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (col + t < N) out[t] = v[t];
        }
      }
    }
}

template <int BM, int BN, int BK, int TM, int TN, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) void k_gemm(
    int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda, const float* __restrict__ B,
    int64_t ldb, float* __restrict__ C, int64_t ldc, int tiles_n, int off32) {
  gemm_tile<BM, BN, BK, TM, TN, TA, TB, VEC, false>(M, N, K, A, lda, B, ldb, C, ldc, tiles_n, off32);
}

// The fused convention on the VALU: one v_fma_f32 per step of each chain.
template <int BM, int BN, int BK, int TM, int TN, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__((BM / TM) * (BN / TN)) void k_gemm_fma(
    int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda, const float* __restrict__ B,
    int64_t ldb, float* __restrict__ C, int64_t ldc, int tiles_n, int off32) {
  gemm_tile<BM, BN, BK, TM, TN, TA, TB, VEC, true>(M, N, K, A, lda, B, ldb, C, ldc, tiles_n, off32);
}

// ---------------------------------------------------------------------------
// Matrix-core multiply, VALU add.
//
// v_mfma_f32_32x32x1_2b_f32 with K = 1 computes, for two independent 32x32
// blocks, D = C + a_i * b_j with one rounding.  With C = -0 (the additive
// identity of IEEE addition, which keeps the sign of a zero product) every D
// element is exactly fl(a_i * b_j) under the contract, including the flush
// rule and signed zeros.  The tests check the single step with C = -0
// against the oracle's multiply (products within ulps of +-2^-126, exact
// ties, subnormal operands, overflow, signed zeros), and run this variant's
// GEMM on the same kinds of data.  No sum is formed inside the matrix core: each product then takes
// its place in the output's own chain with a v_add_f32, k ascending, so the
// declared order is unchanged while the multiplies leave the VALU.
//
// Lane / register layout of the instruction (per block b = 0, 1): A values
// come from lanes 32b..32b+31 (row i = lane - 32b), B values from the same
// lanes (column j = lane - 32b); D[i][j] of block b sits in lane
// j + 32 * ((i / 4) % 2), register 16b + 4 * (i / 8) + i % 4.
//
// Wave tile 64 x 64: lanes 0..63 supply rows 0..63 (block 0 = rows 0..31,
// block 1 = rows 32..63), both halves of the wave supply the same 32
// columns, and two instructions cover columns 0..31 and 32..63.  The
// workgroup is 2 x 2 waves, a 128 x 128 output tile, with BK-deep k slabs
// staged through LDS exactly as in the VALU kernel.
typedef float floatx32 __attribute__((ext_vector_type(32)));

template <int BK, bool TA, bool TB, bool VEC, bool FUSED>
__device__ __forceinline__ void gemm_mfma_tile(int64_t M, int64_t N, int64_t K, const float* __restrict__ A,
                                               int64_t lda, const float* __restrict__ B, int64_t ldb,
                                               float* __restrict__ C, int64_t ldc, int tiles_n, int off32) {
  constexpr int BM = 128, BN = 128, NT = 256;
  // A transposing store puts a wave's 64 lanes on 8 k rows, 4 apart, and 8
  // consecutive words of each: rows of 130 floats spread them over distinct
  // banks (rows of 132 put pairs of them on one; measured 2% faster on the
  // forward workload, same bits).
  using S = SlabStager<BM, BN, BK, NT, TA, TB, VEC, (TA ? 4 : 2), (TB ? 2 : 4)>;
  __shared__ __attribute__((aligned(16))) typename S::ASlab As[2];
  __shared__ __attribute__((aligned(16))) typename S::BSlab Bs[2];

  const int tile = blockIdx.x;
  const int64_t i0 = (int64_t)(tile / tiles_n) * BM;
  const int64_t j0 = (int64_t)(tile % tiles_n) * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * 64;  // wave's first row inside the tile
  const int wn = (wave & 1) * 64;   // wave's first column inside the tile
  S st(As, Bs, A, lda, B, ldb, M, N, K, i0, j0, tid);

  floatx32 acc0, acc1, negz;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    acc0[r] = 0.0f;  // every chain starts at +0
    acc1[r] = 0.0f;
    negz[r] = -0.0f;
  }
  // One k step on operands already in registers.
  auto mfma_step = [&](float a, float b0, float b1) __attribute__((always_inline)) {
    if constexpr (FUSED) {
      // The chain value is the C operand: acc = fl(a * b + acc), one rounding.
      acc0 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b1, acc1, 0, 0, 0);
    } else {
      const floatx32 p0 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b0, negz, 0, 0, 0);
      const floatx32 p1 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b1, negz, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 32; ++r) acc0[r] = acc0[r] + p0[r];
#pragma unroll
      for (int r = 0; r < 32; ++r) acc1[r] = acc1[r] + p1[r];
    }
  };
  auto mac_step = [&](int buf, int kk) __attribute__((always_inline)) {
    mfma_step(As[buf][kk][wm + lane], Bs[buf][kk][wn + (lane & 31)], Bs[buf][kk][wn + 32 + (lane & 31)]);
  };
  // A full slab: the operands of step kk + 1 are read from LDS before the
  // matrix instructions of step kk are issued (held in place by scheduling
  // barriers), so the matrix pipe does not wait on LDS latency between steps.
  auto full_slab = [&](int buf) __attribute__((always_inline)) {
    float op[2][3];
    op[0][0] = As[buf][0][wm + lane];
    op[0][1] = Bs[buf][0][wn + (lane & 31)];
    op[0][2] = Bs[buf][0][wn + 32 + (lane & 31)];
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      if (kk + 1 < BK) {
        const int nx = (kk + 1) & 1;
        op[nx][0] = As[buf][kk + 1][wm + lane];
        op[nx][1] = Bs[buf][kk + 1][wn + (lane & 31)];
        op[nx][2] = Bs[buf][kk + 1][wn + 32 + (lane & 31)];
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_step(op[kk & 1][0], op[kk & 1][1], op[kk & 1][2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const bool interior = VEC && off32 && i0 + BM <= M && j0 + BN <= N;
  run_k_loop<BK>(st, interior, K, full_slab, mac_step);

  // Register r of a lane holds row 32*(r/16) + 8*((r%16)/4) + 4*(lane/32) + r%4
  // of the wave tile, column lane%32 (+32 for the second instruction).
  const int64_t col0 = j0 + wn + (lane & 31);
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const int rr = r & 15;
    const int64_t row = i0 + wm + 32 * (r >> 4) + 8 * (rr >> 2) + 4 * (lane >> 5) + (rr & 3);
    if (row < M) {
      if (col0 < N) C[row * ldc + col0] = acc0[r];
      if (col0 + 32 < N) C[row * ldc + col0 + 32] = acc1[r];
    }
  }
}

template <int BK, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(256) void k_gemm_mfma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A,
                                                   int64_t lda, const float* __restrict__ B, int64_t ldb,
                                                   float* __restrict__ C, int64_t ldc, int tiles_n, int off32) {
  gemm_mfma_tile<BK, TA, TB, VEC, false>(M, N, K, A, lda, B, ldb, C, ldc, tiles_n, off32);
}

// The fused convention on the matrix cores: v_mfma_f32_32x32x1_2b_f32 with
// K = 1 and the chain as C is one fused multiply-add per output per step, so
// consecutive instructions over ascending k form exactly the serial fused
// chain of every output, with no VALU arithmetic at all.
template <int BK, bool TA, bool TB, bool VEC>
__global__ __launch_bounds__(256) void k_gemm_mfma_fma(int64_t M, int64_t N, int64_t K,
                                                       const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb,
                                                       float* __restrict__ C, int64_t ldc, int tiles_n,
                                                       int off32) {
  gemm_mfma_tile<BK, TA, TB, VEC, true>(M, N, K, A, lda, B, ldb, C, ldc, tiles_n, off32);
}

template <int BK, bool TA, bool TB, bool VEC, bool FUSED>
hipError_t launch_mfma(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                       float* C, int64_t ldc, hipStream_t stream) {
  const int64_t tiles_m = (M + 127) / 128;
  const int64_t tiles_n = (N + 127) / 128;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const int off32 = slab_offsets_fit<128, 128, BK, TA, TB>(lda, ldb) ? 1 : 0;
  if constexpr (FUSED)
    hipLaunchKernelGGL((k_gemm_mfma_fma<BK, TA, TB, VEC>), dim3((unsigned)tiles), dim3(256), 0, stream, M, N, K, A,
                       lda, B, ldb, C, ldc, (int)tiles_n, off32);
  else
    hipLaunchKernelGGL((k_gemm_mfma<BK, TA, TB, VEC>), dim3((unsigned)tiles), dim3(256), 0, stream, M, N, K, A,
                       lda, B, ldb, C, ldc, (int)tiles_n, off32);
  return hipGetLastError();
}

// 32-deep k slabs: half the barriers and slab loads per MAC of 16-deep
// ones; measured on MI355X 4-5% faster for the fused chains and 1% for the
// products-plus-VALU-adds kernel (220 VGPRs: still two waves per SIMD).
template <bool FUSED>
hipError_t dispatch_mfma(int ta, int tb, bool vec, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                         const float* B, int64_t ldb, float* C, int64_t ldc, hipStream_t stream) {
#define REPRO_GEMM_CASE(TA_, TB_)                                                                     \
  if (ta == TA_ && tb == TB_)                                                                         \
    return vec ? launch_mfma<32, TA_, TB_, true, FUSED>(M, N, K, A, lda, B, ldb, C, ldc, stream) \
               : launch_mfma<32, TA_, TB_, false, FUSED>(M, N, K, A, lda, B, ldb, C, ldc, stream);
  REPRO_GEMM_CASE(0, 0)
  REPRO_GEMM_CASE(1, 0)
  REPRO_GEMM_CASE(0, 1)
  REPRO_GEMM_CASE(1, 1)
#undef REPRO_GEMM_CASE
  return hipErrorInvalidValue;
}

template <int BM, int BN, int BK, int TM, int TN, bool TA, bool TB, bool VEC, bool FUSED>
hipError_t launch_tiled(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                        int64_t ldb, float* C, int64_t ldc, hipStream_t stream) {
  using T = GemmTile<BM, BN, BK, TM, TN, TA, TB, VEC>;
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t tiles_n = (N + BN - 1) / BN;
  const int64_t tiles = tiles_m * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  // Interior tiles address slabs with 32-bit lane offsets when they fit.
  const int off32 = slab_offsets_fit<BM, BN, BK, TA, TB>(lda, ldb) ? 1 : 0;
  if constexpr (FUSED)
    hipLaunchKernelGGL((k_gemm_fma<BM, BN, BK, TM, TN, TA, TB, VEC>), dim3((unsigned)tiles), dim3(T::NT), 0,
                       stream, M, N, K, A, lda, B, ldb, C, ldc, (int)tiles_n, off32);
  else
    hipLaunchKernelGGL((k_gemm<BM, BN, BK, TM, TN, TA, TB, VEC>), dim3((unsigned)tiles), dim3(T::NT), 0, stream,
                       M, N, K, A, lda, B, ldb, C, ldc, (int)tiles_n, off32);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int TM, int TN, bool FUSED>
hipError_t dispatch(int ta, int tb, bool vec, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                    const float* B, int64_t ldb, float* C, int64_t ldc, hipStream_t stream) {
#define REPRO_GEMM_CASE(TA_, TB_)                                                                             \
  if (ta == TA_ && tb == TB_)                                                                                 \
    return vec ? launch_tiled<BM, BN, BK, TM, TN, TA_, TB_, true, FUSED>(M, N, K, A, lda, B, ldb, C, ldc,     \
                                                                         stream)                              \
               : launch_tiled<BM, BN, BK, TM, TN, TA_, TB_, false, FUSED>(M, N, K, A, lda, B, ldb, C, ldc,    \
                                                                          stream);
  REPRO_GEMM_CASE(0, 0)
  REPRO_GEMM_CASE(1, 0)
  REPRO_GEMM_CASE(0, 1)
  REPRO_GEMM_CASE(1, 1)
#undef REPRO_GEMM_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                       const float* B, int64_t ldb, float* C, int64_t ldc, int variant, bool fused,
                       hipStream_t stream) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  // 16-byte loads need aligned bases, leading dimensions that keep rows
  // aligned, and a contiguous extent that is a multiple of 4 so that a
  // chunk is either wholly inside or wholly outside the matrix.
  const int64_t a_contig = trans_a ? M : K;
  const int64_t b_contig = trans_b ? K : N;
  // (Variant 1 of the unfused kernels forces scalar loads; the fused
  // variants always take 16-byte loads when they can.)
  const bool vec = (fused || variant != 1) && al16(A) && al16(B) && lda % 4 == 0 && ldb % 4 == 0 &&
                   a_contig % 4 == 0 && b_contig % 4 == 0;
  if (fused) {  // variant 0: matrix cores, 1: VALU v_fma_f32
    if (variant == 0)
      return dispatch_mfma<true>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
    // The same tiles as the unfused VALU kernel (variant 4): 256 x 128 for
    // large outputs (measured 4-5% faster than 128 x 128 on both
    // workloads), else 128 x 128 with 32-deep slabs.
    if (((M + 255) / 256) * ((N + 127) / 128) >= 512)
      return dispatch<256, 128, 16, 16, 8, true>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
    return dispatch<128, 128, 32, 8, 8, true>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
  }
  // Variant 0, the default, and variant 3: products on the matrix cores,
  // adds on the VALU (k_gemm_mfma).  The matrix cores and the VALU take
  // turns on this chip, so per MAC this costs what the VALU's multiply and
  // add cost; but with half the VALU instructions the kernel runs at a
  // higher clock, and measured on MI355X it is 1-6% faster than the VALU
  // kernel on the two GEMM workloads, with the same bits.
  if (variant == 0 || variant == 3)
    return dispatch_mfma<false>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
  if (variant == 2)
    return dispatch<64, 64, 16, 4, 4, false>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
  // Variant 4, the VALU multiply and add, on large outputs: 256 x 128 tiles,
  // 16 x 8 outputs per lane, 16-deep slabs (250 VGPRs: two waves per SIMD;
  // 50 KB of LDS).  Each k step reads 24 values from LDS for 128 MACs
  // instead of 16 for 64, and each slab moves half as many A and B bytes per
  // MAC; measured on MI355X 3-4% faster than 128 x 128 tiles on both GEMM
  // workloads, same bits.  Used when there are at least two such tiles per
  // CU, so the larger tile costs no parallelism.
  if (variant == 4 && ((M + 255) / 256) * ((N + 127) / 128) >= 512)
    return dispatch<256, 128, 16, 16, 8, false>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
  // Otherwise (variant 1, and variant 4 on smaller outputs) 128 x 128 tiles
  // with 32-deep k slabs: half the barriers and slab loads per MAC of
  // 16-deep ones; measured on MI355X 2% faster on the weight-gradient
  // workload and 1-10% on the forward one, same bits (two waves per SIMD;
  // 67.6 KB of LDS: two workgroups per CU).
  return dispatch<128, 128, 32, 8, 8, false>(trans_a, trans_b, vec, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

}  // namespace repro
