// Measurement support for the ALU rooflines (not part of the reproducible
// operations): the VALU issue rate of gfx950 for single-instruction streams
// and for the interleavings that the kernels' instruction mixes contain, and
// whether matrix-core instructions issue alongside VALU work on one SIMD.
//
// Each stream is a loop body of 128 to 260 independent instructions
// (sources v0..v15, results v16..v47, no dependences between them); a workgroup of
// 256 lanes puts one wave on each SIMD of its CU, and a launch of
// 256 x W workgroups puts W waves on every SIMD.  The rate is wave-
// instructions per SIMD per shader clock over the launch's event time, with
// the clock taken inside the kernel from s_memtime (shader clock) against
// s_memrealtime (100 MHz).  Built into its own library, libvalu_rates.so,
// which only bench.py --valu-rates loads.
#include <hip/hip_runtime.h>

#include <vector>

namespace {

// Streams: the instruction text of one pass of the loop body.
#define R8(x) x x x x x x x x
#define XOR8 \
  "v_xor_b32_e32 v16, v0, v1\n" "v_xor_b32_e32 v17, v2, v3\n" "v_xor_b32_e32 v18, v4, v5\n" \
  "v_xor_b32_e32 v19, v6, v7\n" "v_xor_b32_e32 v20, v8, v9\n" "v_xor_b32_e32 v21, v10, v11\n" \
  "v_xor_b32_e32 v22, v12, v13\n" "v_xor_b32_e32 v23, v14, v15\n"
#define XOR64_8 \
  "v_xor_b32_e64 v16, v0, v1\n" "v_xor_b32_e64 v17, v2, v3\n" "v_xor_b32_e64 v18, v4, v5\n" \
  "v_xor_b32_e64 v19, v6, v7\n" "v_xor_b32_e64 v20, v8, v9\n" "v_xor_b32_e64 v21, v10, v11\n" \
  "v_xor_b32_e64 v22, v12, v13\n" "v_xor_b32_e64 v23, v14, v15\n"
#define MUL8 \
  "v_mul_f32_e32 v16, v0, v1\n" "v_mul_f32_e32 v17, v2, v3\n" "v_mul_f32_e32 v18, v4, v5\n" \
  "v_mul_f32_e32 v19, v6, v7\n" "v_mul_f32_e32 v20, v8, v9\n" "v_mul_f32_e32 v21, v10, v11\n" \
  "v_mul_f32_e32 v22, v12, v13\n" "v_mul_f32_e32 v23, v14, v15\n"
#define ALIGN8 \
  "v_alignbit_b32 v24, v0, v1, 24\n" "v_alignbit_b32 v25, v2, v3, 24\n" "v_alignbit_b32 v26, v4, v5, 24\n" \
  "v_alignbit_b32 v27, v6, v7, 24\n" "v_alignbit_b32 v28, v8, v9, 24\n" "v_alignbit_b32 v29, v10, v11, 24\n" \
  "v_alignbit_b32 v30, v12, v13, 24\n" "v_alignbit_b32 v31, v14, v15, 24\n"
#define ADD64_8 \
  "v_lshl_add_u64 v[32:33], v[0:1], 0, v[2:3]\n" "v_lshl_add_u64 v[34:35], v[4:5], 0, v[6:7]\n" \
  "v_lshl_add_u64 v[36:37], v[8:9], 0, v[10:11]\n" "v_lshl_add_u64 v[38:39], v[12:13], 0, v[14:15]\n" \
  "v_lshl_add_u64 v[40:41], v[2:3], 0, v[4:5]\n" "v_lshl_add_u64 v[42:43], v[6:7], 0, v[8:9]\n" \
  "v_lshl_add_u64 v[44:45], v[10:11], 0, v[12:13]\n" "v_lshl_add_u64 v[46:47], v[14:15], 0, v[0:1]\n"
#define SHL8 \
  "v_lshlrev_b32_e32 v16, 8, v0\n" "v_lshlrev_b32_e32 v17, 8, v2\n" "v_lshlrev_b32_e32 v18, 8, v4\n" \
  "v_lshlrev_b32_e32 v19, 8, v6\n" "v_lshlrev_b32_e32 v20, 8, v8\n" "v_lshlrev_b32_e32 v21, 8, v10\n" \
  "v_lshlrev_b32_e32 v22, 8, v12\n" "v_lshlrev_b32_e32 v23, 8, v14\n"
#define SHR8 \
  "v_lshrrev_b32_e32 v16, 8, v0\n" "v_lshrrev_b32_e32 v17, 8, v2\n" "v_lshrrev_b32_e32 v18, 8, v4\n" \
  "v_lshrrev_b32_e32 v19, 8, v6\n" "v_lshrrev_b32_e32 v20, 8, v8\n" "v_lshrrev_b32_e32 v21, 8, v10\n" \
  "v_lshrrev_b32_e32 v22, 8, v12\n" "v_lshrrev_b32_e32 v23, 8, v14\n"
#define ALT8 \
  "v_alignbit_b32 v24, v0, v1, 24\n" "v_xor_b32_e32 v17, v2, v3\n" "v_alignbit_b32 v26, v4, v5, 24\n" \
  "v_xor_b32_e32 v19, v6, v7\n" "v_alignbit_b32 v28, v8, v9, 24\n" "v_xor_b32_e32 v21, v10, v11\n" \
  "v_alignbit_b32 v30, v12, v13, 24\n" "v_xor_b32_e32 v23, v14, v15\n"
#define ONE_IN_65 R8(XOR8) "v_alignbit_b32 v24, v0, v1, 24\n"
#define ALIGN4 \
  "v_alignbit_b32 v24, v0, v1, 24\n" "v_alignbit_b32 v25, v2, v3, 24\n" "v_alignbit_b32 v26, v4, v5, 24\n" \
  "v_alignbit_b32 v27, v6, v7, 24\n"
#define XOR4 \
  "v_xor_b32_e32 v16, v0, v1\n" "v_xor_b32_e32 v17, v2, v3\n" "v_xor_b32_e32 v18, v4, v5\n" \
  "v_xor_b32_e32 v19, v6, v7\n"
// The G function's mix: 6 64-bit adds and 6 alignbits (half-rate) beside
// 8 xors (full-rate), clustered by kind.
#define G_MIX \
  "v_lshl_add_u64 v[32:33], v[0:1], 0, v[2:3]\n" "v_lshl_add_u64 v[34:35], v[4:5], 0, v[6:7]\n" \
  "v_lshl_add_u64 v[36:37], v[8:9], 0, v[10:11]\n" "v_lshl_add_u64 v[38:39], v[12:13], 0, v[14:15]\n" \
  "v_lshl_add_u64 v[40:41], v[2:3], 0, v[4:5]\n" "v_lshl_add_u64 v[42:43], v[6:7], 0, v[8:9]\n" \
  "v_alignbit_b32 v24, v0, v1, 24\n" "v_alignbit_b32 v25, v2, v3, 24\n" "v_alignbit_b32 v26, v4, v5, 24\n" \
  "v_alignbit_b32 v27, v6, v7, 24\n" "v_alignbit_b32 v28, v8, v9, 24\n" "v_alignbit_b32 v29, v10, v11, 24\n" \
  XOR8

constexpr int kStreams = 14;
// Instructions per pass of each stream's loop body.
constexpr int kPassLength[kStreams] = {128, 128, 128, 128, 128, 128, 128, 128, 260, 130, 128, 128, 128, 160};

#define CLOBBERS                                                                                              \
  "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23", "v24", "v25", "v26", "v27", "v28", "v29", "v30", \
      "v31", "v32", "v33", "v34", "v35", "v36", "v37", "v38", "v39", "v40", "v41", "v42", "v43", "v44", "v45", \
      "v46", "v47"

template <int S>
__device__ __forceinline__ void pass() {
  if constexpr (S == 0) asm volatile(R8(MUL8) R8(MUL8) ::: CLOBBERS);
  if constexpr (S == 1) asm volatile(R8(XOR8) R8(XOR8) ::: CLOBBERS);
  if constexpr (S == 2) asm volatile(R8(XOR64_8) R8(XOR64_8) ::: CLOBBERS);
  if constexpr (S == 3) asm volatile(R8(ALIGN8) R8(ALIGN8) ::: CLOBBERS);
  if constexpr (S == 4) asm volatile(R8(ADD64_8) R8(ADD64_8) ::: CLOBBERS);
  if constexpr (S == 5) asm volatile(R8(SHL8) R8(SHL8) ::: CLOBBERS);
  if constexpr (S == 6) asm volatile(R8(SHR8) R8(SHR8) ::: CLOBBERS);
  if constexpr (S == 7) asm volatile(R8(ALT8) R8(ALT8) ::: CLOBBERS);
  // Four v_alignbit_b32 after 256 xors: a short cluster of half-rate
  // instructions in a long full-rate run.
  if constexpr (S == 8) asm volatile(R8(XOR8) R8(XOR8) R8(XOR8) R8(XOR8) "v_alignbit_b32 v24, v0, v1, 24\n"
                                     "v_alignbit_b32 v25, v2, v3, 24\n" "v_alignbit_b32 v26, v4, v5, 24\n"
                                     "v_alignbit_b32 v27, v6, v7, 24\n" ::: CLOBBERS);
  // One v_alignbit_b32 per 65 instructions.
  if constexpr (S == 9) asm volatile(ONE_IN_65 ONE_IN_65 ::: CLOBBERS);
  // Long runs of each kind: 64 v_alignbit_b32, then 64 v_xor_b32.
  if constexpr (S == 10) asm volatile(R8(ALIGN8) R8(XOR8) ::: CLOBBERS);
  // One half-rate instruction in four, clustered: 4 v_alignbit_b32, 12 v_xor_b32.
  if constexpr (S == 11) asm volatile(R8(ALIGN4 XOR4 XOR4 XOR4) ::: CLOBBERS);
  // 8 v_lshl_add_u64, then 8 v_xor_b32.
  if constexpr (S == 12) asm volatile(ADD64_8 XOR8 ADD64_8 XOR8 ADD64_8 XOR8 ADD64_8 XOR8 ADD64_8 XOR8 ADD64_8 XOR8
                                          ADD64_8 XOR8 ADD64_8 XOR8 ::: CLOBBERS);
  // The G function's mix, clustered by kind (20 instructions, 12 half-rate).
  if constexpr (S == 13) asm volatile(R8(G_MIX) ::: CLOBBERS);
}

template <int S>
__global__ __launch_bounds__(256) void k_valu_stream(float* __restrict__ out, long long* __restrict__ meta,
                                                     int iters) {
  // Distinct, finite operand values in v0..v15.
  asm volatile(
      "v_cvt_f32_u32 v0, 1\n v_cvt_f32_u32 v1, 2\n v_cvt_f32_u32 v2, 3\n v_cvt_f32_u32 v3, 5\n"
      "v_cvt_f32_u32 v4, 7\n v_cvt_f32_u32 v5, 11\n v_cvt_f32_u32 v6, 13\n v_cvt_f32_u32 v7, 17\n"
      "v_cvt_f32_u32 v8, 19\n v_cvt_f32_u32 v9, 23\n v_cvt_f32_u32 v10, 29\n v_cvt_f32_u32 v11, 31\n"
      "v_cvt_f32_u32 v12, 37\n v_cvt_f32_u32 v13, 41\n v_cvt_f32_u32 v14, 43\n v_cvt_f32_u32 v15, 47\n" ::
          : "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15");
  const long long t0 = __builtin_amdgcn_s_memtime();
  const long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) pass<S>();
  const long long t1 = __builtin_amdgcn_s_memtime();
  const long long r1 = __builtin_amdgcn_s_memrealtime();
  float keep;
  asm volatile("v_mov_b32 %0, v16" : "=v"(keep)::"v16");
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = keep;
  if (threadIdx.x % 64 == 0) {
    const size_t w = (size_t)blockIdx.x * 4 + threadIdx.x / 64;
    meta[2 * w] = t1 - t0;
    meta[2 * w + 1] = r1 - r0;
  }
}

// Co-issue of matrix-core instructions with VALU adds on one SIMD.  A
// 512-lane workgroup has 8 waves and wave w runs on SIMD w % 4, so waves 0-3
// (matrix role) and waves 4-7 (VALU role) pair up, one of each per SIMD.
// The matrix role runs 4 independent accumulating chains (fp32
// v_mfma_f32_32x32x1_2b_f32, or bf16 v_mfma_f32_32x32x8_bf16); the VALU role
// runs the v_add_f32 stream.  MODE 0 runs both roles, 1 only the matrix role,
// 2 only the VALU role (the other waves exit at once).
typedef float v32f __attribute__((ext_vector_type(32)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
#define ADD8 \
  "v_add_f32_e32 v16, v0, v1\n" "v_add_f32_e32 v17, v2, v3\n" "v_add_f32_e32 v18, v4, v5\n" \
  "v_add_f32_e32 v19, v6, v7\n" "v_add_f32_e32 v20, v8, v9\n" "v_add_f32_e32 v21, v10, v11\n" \
  "v_add_f32_e32 v22, v12, v13\n" "v_add_f32_e32 v23, v14, v15\n"

template <int KIND, int MODE>
__global__ __launch_bounds__(512) void k_coissue(float* __restrict__ out, int iters_m, int iters_v) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  float r = 0.0f;
  if (wave < 4) {
    if (MODE == 2) return;
    if constexpr (KIND == 0) {
      const float a = 1.0f + lane, b = 0.5f - lane;
      v32f c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int it = 0; it < iters_m; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x1f32(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x1f32(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x1f32(b, b, c3, 0, 0, 0);
      }
      for (int i = 0; i < 32; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
    } else {
      const v4s a = {(short)lane, 0x3f80, 0x3f00, 0x4000}, b = {0x3f80, (short)lane, 0x3e80, 0x3f80};
      v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int it = 0; it < iters_m; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(b, b, c3, 0, 0, 0);
      }
      for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
    }
  } else {
    if (MODE == 1) return;
    asm volatile(
        "v_cvt_f32_u32 v0, 1\n v_cvt_f32_u32 v1, 2\n v_cvt_f32_u32 v2, 3\n v_cvt_f32_u32 v3, 5\n"
        "v_cvt_f32_u32 v4, 7\n v_cvt_f32_u32 v5, 11\n v_cvt_f32_u32 v6, 13\n v_cvt_f32_u32 v7, 17\n"
        "v_cvt_f32_u32 v8, 19\n v_cvt_f32_u32 v9, 23\n v_cvt_f32_u32 v10, 29\n v_cvt_f32_u32 v11, 31\n"
        "v_cvt_f32_u32 v12, 37\n v_cvt_f32_u32 v13, 41\n v_cvt_f32_u32 v14, 43\n v_cvt_f32_u32 v15, 47\n" ::
            : "v0", "v1", "v2", "v3", "v4", "v5", "v6", "v7", "v8", "v9", "v10", "v11", "v12", "v13", "v14", "v15");
    for (int it = 0; it < iters_v; ++it)
      asm volatile(R8(ADD8) R8(ADD8)::: "v16", "v17", "v18", "v19", "v20", "v21", "v22", "v23");
    asm volatile("v_mov_b32 %0, v16" : "=v"(r)::"v16");
  }
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = r;
}

typedef void (*CoissueKernel)(float*, int, int);
constexpr CoissueKernel kCoissue[2][3] = {{k_coissue<0, 0>, k_coissue<0, 1>, k_coissue<0, 2>},
                                          {k_coissue<1, 0>, k_coissue<1, 1>, k_coissue<1, 2>}};

typedef void (*StreamKernel)(float*, long long*, int);
constexpr StreamKernel kKernels[kStreams] = {k_valu_stream<0>,  k_valu_stream<1>,  k_valu_stream<2>,  k_valu_stream<3>,
                                             k_valu_stream<4>,  k_valu_stream<5>,  k_valu_stream<6>,  k_valu_stream<7>,
                                             k_valu_stream<8>,  k_valu_stream<9>,  k_valu_stream<10>, k_valu_stream<11>,
                                             k_valu_stream<12>, k_valu_stream<13>};

}  // namespace

extern "C" {

// Number of streams and the name of stream `s` (nullptr when out of range).
int valu_rates_count() { return kStreams; }
const char* valu_rates_name(int s) {
  static const char* const names[kStreams] = {"v_mul_f32_e32",
                                              "v_xor_b32_e32",
                                              "v_xor_b32_e64 (8-byte encoding)",
                                              "v_alignbit_b32",
                                              "v_lshl_add_u64",
                                              "v_lshlrev_b32_e32",
                                              "v_lshrrev_b32_e32",
                                              "v_alignbit_b32 and v_xor_b32_e32 alternating",
                                              "4 v_alignbit_b32 after 256 v_xor_b32_e32",
                                              "1 v_alignbit_b32 per 65 instructions",
                                              "64 v_alignbit_b32 then 64 v_xor_b32_e32",
                                              "4 v_alignbit_b32 then 12 v_xor_b32_e32",
                                              "8 v_lshl_add_u64 then 8 v_xor_b32_e32",
                                              "G mix: 6 v_lshl_add_u64, 6 v_alignbit_b32, 8 v_xor_b32_e32"};
  return s >= 0 && s < kStreams ? names[s] : nullptr;
}

// Runs stream `s` with `waves_per_simd` (1..8) waves on every SIMD of a
// 256-CU device for `iters` passes; writes {wave-instructions per SIMD per
// shader clock, shader clock in GHz, event milliseconds}.  Returns 0, or -1
// for bad arguments, -2 for a HIP error.
int valu_rates_run(int s, int waves_per_simd, int iters, double* result) {
  if (s < 0 || s >= kStreams || waves_per_simd < 1 || waves_per_simd > 8 || iters < 1 || result == nullptr)
    return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return -2;
  const int blocks = cus * waves_per_simd;
  float* out = nullptr;
  long long* meta = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -2;
  if (hipMalloc(&out, sizeof(float) * 256 * (size_t)blocks) == hipSuccess &&
      hipMalloc(&meta, sizeof(long long) * 8 * (size_t)blocks) == hipSuccess && hipEventCreate(&e0) == hipSuccess &&
      hipEventCreate(&e1) == hipSuccess) {
    hipLaunchKernelGGL(kKernels[s], dim3(blocks), dim3(256), 0, 0, out, meta, 16);
    const hipError_t warm = hipGetLastError();
    (void)hipEventRecord(e0, 0);
    hipLaunchKernelGGL(kKernels[s], dim3(blocks), dim3(256), 0, 0, out, meta, iters);
    const hipError_t timed = hipGetLastError();
    (void)hipEventRecord(e1, 0);
    float ms = 0.f;
    std::vector<long long> h(8 * (size_t)blocks);
    if (warm == hipSuccess && timed == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
        hipEventElapsedTime(&ms, e0, e1) == hipSuccess &&
        hipMemcpy(h.data(), meta, sizeof(long long) * h.size(), hipMemcpyDeviceToHost) == hipSuccess && ms > 0.f) {
      double cyc = 0, rt = 0;
      for (size_t w = 0; w < 4 * (size_t)blocks; ++w) {
        cyc += (double)h[2 * w];
        rt += (double)h[2 * w + 1];
      }
      const double ghz = rt > 0 ? cyc / rt * 0.1 : 0.0;
      const double instr = (double)iters * kPassLength[s] * 4.0 * blocks;  // wave-instructions
      result[0] = ghz > 0 ? instr / (4.0 * cus) / (ms * 1e-3 * ghz * 1e9) : 0.0;
      result[1] = ghz;
      result[2] = ms;
      rc = 0;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  if (meta) (void)hipFree(meta);
  return rc;
}

// Event milliseconds of the co-issue kernel for matrix kind `kind` (0 fp32,
// 1 bf16) in each mode: result[0] both roles, [1] the matrix role alone,
// [2] the VALU role alone.  One 512-lane workgroup per CU; the matrix role
// runs `iters_m` passes of 4 instructions, the VALU role `iters_v` passes of
// 128 adds.  Returns 0, or -1 for bad arguments, -2 for a HIP error.
int valu_rates_coissue(int kind, int iters_m, int iters_v, double* result) {
  if (kind < 0 || kind > 1 || iters_m < 1 || iters_v < 1 || result == nullptr) return -1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return -2;
  float* out = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = -2;
  if (hipMalloc(&out, sizeof(float) * 512 * (size_t)cus) == hipSuccess && hipEventCreate(&e0) == hipSuccess &&
      hipEventCreate(&e1) == hipSuccess) {
    rc = 0;
    for (int mode = 0; mode < 3 && rc == 0; ++mode) {
      hipLaunchKernelGGL(kCoissue[kind][mode], dim3(cus), dim3(512), 0, 0, out, 16, 16);
      const hipError_t warm = hipGetLastError();
      (void)hipEventRecord(e0, 0);
      hipLaunchKernelGGL(kCoissue[kind][mode], dim3(cus), dim3(512), 0, 0, out, iters_m, iters_v);
      const hipError_t timed = hipGetLastError();
      (void)hipEventRecord(e1, 0);
      float ms = 0.f;
      if (warm != hipSuccess || timed != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
          hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f)
        rc = -2;
      result[mode] = ms;
    }
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (out) (void)hipFree(out);
  return rc;
}

}  // extern "C"
