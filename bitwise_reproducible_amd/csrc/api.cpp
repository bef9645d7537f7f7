// C-ABI front end of librepro.so: argument checks, the host-side scalars,
// and the kernel launches.  See include/repro.h for the contract of every
// entry point.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <xmmintrin.h>

#include <mutex>
#include <vector>

#include "internal.h"
#include "repro.h"

// The host-side scalars below change the SSE control register around their
// arithmetic; declaring access to the floating-point environment keeps the
// compiler from moving that arithmetic across the change.  (The device pass,
// which sees only the no-allocation workspace array below, does not know the
// pragma.)
#ifndef __HIP_DEVICE_COMPILE__
#pragma STDC FENV_ACCESS ON
#endif

namespace {

using repro::AdamwScalars;
using repro::ReplicaPtrs;

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? REPRO_OK : REPRO_EDEVICE; }

// Host binary32 arithmetic under the contract of repro.h: the SSE control
// register is set to round-to-nearest with FTZ and DAZ on for the duration
// (the x86 definition of the flush rule), and restored afterwards.
class HostFp32 {
 public:
  HostFp32() : saved_(_mm_getcsr()) { _mm_setcsr((saved_ & ~0x6000u) | 0x8000u | 0x0040u | 0x1F80u); }
  ~HostFp32() { _mm_setcsr(saved_); }
  static float sub(float a, float b) { return a - b; }
  static float mul(float a, float b) { return a * b; }
  static float div(float a, float b) { return a / b; }

 private:
  unsigned saved_;
};

// Appendix A.3 reciprocal: fl(1 / R) on the host.
float replica_reciprocal(int R) {
  HostFp32 env;
  return HostFp32::div(1.0f, (float)R);
}

// fl(1 / d) on the host (Appendix A.3).
float reciprocal(int d) {
  HostFp32 env;
  return HostFp32::div(1.0f, (float)d);
}

// AdamW host scalars: c = 1 - beta, beta^step as step-1 serial products, and
// the reciprocals of the bias corrections.
AdamwScalars adamw_scalars(float lr, float beta1, float beta2, float eps, float wd, int64_t step) {
  HostFp32 env;
  AdamwScalars s;
  s.lr = lr;
  s.beta1 = beta1;
  s.beta2 = beta2;
  s.eps = eps;
  s.wd = wd;
  s.c1 = HostFp32::sub(1.0f, s.beta1);
  s.c2 = HostFp32::sub(1.0f, s.beta2);
  float pow1 = s.beta1, pow2 = s.beta2;
  for (int64_t t = 2; t <= step; ++t) {
    pow1 = HostFp32::mul(pow1, s.beta1);
    pow2 = HostFp32::mul(pow2, s.beta2);
  }
  s.r1 = HostFp32::div(1.0f, HostFp32::sub(1.0f, pow1));
  s.r2 = HostFp32::div(1.0f, HostFp32::sub(1.0f, pow2));
  return s;
}

}  // namespace

extern "C" {

const char* repro_spec_version(void) { return "repro-spec-1"; }

const char* repro_strerror(int status) {
  switch (status) {
    case REPRO_OK: return "ok";
    case REPRO_EINVAL: return "invalid argument";
    case REPRO_EALIGN: return "pointer not aligned as the call requires";
    case REPRO_EDEVICE: return "HIP launch or runtime error";
    case REPRO_ESPACE: return "workspace too small";
    default: return "unknown status";
  }
}

namespace {

int gemm_checked(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                 const float* B, int64_t ldb, float* C, int64_t ldc, int32_t variant, bool fused, void* stream) {
  if (M < 0 || N < 0 || K < 0 || variant < 0 || variant > (fused ? 1 : 4)) return REPRO_EINVAL;
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return REPRO_EINVAL;
  if (M == 0 || N == 0) return REPRO_OK;
  if (C == nullptr || ldc < N) return REPRO_EINVAL;
  if (K > 0) {
    if (A == nullptr || B == nullptr) return REPRO_EINVAL;
    if (lda < (trans_a ? M : K) || ldb < (trans_b ? K : N)) return REPRO_EINVAL;
    if (!aligned4(A) || !aligned4(B)) return REPRO_EALIGN;
  }
  if (!aligned4(C)) return REPRO_EALIGN;
  return status_of(repro::launch_gemm(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, variant, fused,
                                      static_cast<hipStream_t>(stream)));
}

}  // namespace

int repro_gemm_variant(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                       const float* B, int64_t ldb, float* C, int64_t ldc, int32_t variant, void* stream) {
  return gemm_checked(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, variant, false, stream);
}

int repro_gemm_fma(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                   const float* B, int64_t ldb, float* C, int64_t ldc, int32_t variant, void* stream) {
  return gemm_checked(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, variant, true, stream);
}

int repro_gemm(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
               const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
  return repro_gemm_variant(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, 0, stream);
}

int repro_tree_reduce_variant(const float* const* replicas, int32_t R, int64_t n, float* out, int32_t average,
                              int32_t variant, void* stream) {
  if (replicas == nullptr || R < 1 || R > REPRO_MAX_REPLICAS || n < 0 || variant < 0 || variant > 2)
    return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (out == nullptr) return REPRO_EINVAL;
  ReplicaPtrs reps = {};
  for (int r = 0; r < R; ++r) {
    if (replicas[r] == nullptr) return REPRO_EINVAL;
    if (!aligned4(replicas[r])) return REPRO_EALIGN;
    reps.p[r] = replicas[r];
  }
  if (!aligned4(out)) return REPRO_EALIGN;
  const float rR = replica_reciprocal(R);
  return status_of(repro::launch_tree_reduce(reps, R, n, out, average != 0, rR, variant,
                                             static_cast<hipStream_t>(stream)));
}

int repro_tree_reduce(const float* const* replicas, int32_t R, int64_t n, float* out, int32_t average,
                      void* stream) {
  return repro_tree_reduce_variant(replicas, R, n, out, average, 0, stream);
}

int repro_replay_reduce(const float* const* grads, int32_t dp_replicate, int32_t dp_shard, int32_t accum,
                        int64_t n, float* out, void* stream) {
  if (grads == nullptr || dp_replicate < 1 || dp_replicate > REPRO_MAX_REPLICAS || dp_shard < 1 || accum < 1 ||
      n < 0)
    return REPRO_EINVAL;
  // Each factor is bounded before the product is formed, so it cannot wrap.
  if (dp_shard > REPRO_MAX_REPLAY_BUFFERS || accum > REPRO_MAX_REPLAY_BUFFERS) return REPRO_EINVAL;
  const int64_t nbuf = (int64_t)dp_replicate * dp_shard * accum;
  if (nbuf > REPRO_MAX_REPLAY_BUFFERS) return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (out == nullptr) return REPRO_EINVAL;
  repro::ReplayPtrs a = {};
  for (int64_t b = 0; b < nbuf; ++b) {
    if (grads[b] == nullptr) return REPRO_EINVAL;
    if (!aligned4(grads[b])) return REPRO_EALIGN;
    a.p[b] = grads[b];
  }
  if (!aligned4(out)) return REPRO_EALIGN;
  return status_of(repro::launch_replay(a, (int)nbuf, dp_replicate, dp_shard, accum, reciprocal(accum),
                                        reciprocal(dp_shard), reciprocal(dp_replicate), n, out,
                                        static_cast<hipStream_t>(stream)));
}

int repro_fold_push(float* const* slots, int32_t pushed, const float* part, int64_t n, void* stream) {
  if (slots == nullptr || pushed < 0 || pushed > 126 || n < 0) return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (part == nullptr) return REPRO_EINVAL;
  const int t = __builtin_ctz(~(unsigned)pushed);
  repro::FoldSlotPtrs sl = {};
  for (int L = 0; L <= t; ++L) {
    if (slots[L] == nullptr) return REPRO_EINVAL;
    if (!aligned4(slots[L])) return REPRO_EALIGN;
    sl.p[L] = slots[L];
  }
  if (!aligned4(part)) return REPRO_EALIGN;
  return status_of(repro::launch_fold_push(sl, t, part, n, static_cast<hipStream_t>(stream)));
}

int repro_fold_result(float* const* slots, int32_t pushed, int64_t n, float* out, int32_t divisor, void* stream) {
  if (slots == nullptr || pushed < 1 || pushed > 127 || n < 0 || divisor < 0) return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (out == nullptr) return REPRO_EINVAL;
  repro::FoldSlotPtrs sl = {};
  for (int L = 0; L < REPRO_FOLD_SLOTS; ++L) {
    if (((pushed >> L) & 1) == 0) continue;
    if (slots[L] == nullptr) return REPRO_EINVAL;
    if (!aligned4(slots[L])) return REPRO_EALIGN;
    sl.p[L] = slots[L];
  }
  if (!aligned4(out)) return REPRO_EALIGN;
  const float r = divisor > 0 ? reciprocal(divisor) : 1.0f;
  return status_of(repro::launch_fold_result(sl, pushed, divisor > 0, r, out, n, static_cast<hipStream_t>(stream)));
}

int repro_adamw_variant(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2, float eps,
                        float weight_decay, int64_t step, int32_t variant, void* stream) {
  if (n < 0 || step < 1 || variant < 0 || variant > 1) return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (state == nullptr || grad == nullptr) return REPRO_EINVAL;
  if (!aligned4(state) || !aligned4(grad)) return REPRO_EALIGN;
  const AdamwScalars s = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step);
  return status_of(repro::launch_adamw(state, grad, n, s, variant, static_cast<hipStream_t>(stream)));
}

int repro_adamw(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2, float eps,
                float weight_decay, int64_t step, void* stream) {
  return repro_adamw_variant(state, grad, n, lr, beta1, beta2, eps, weight_decay, step, 0, stream);
}

namespace {

// A second stream per device and a pool of events, created on first use and
// kept for the life of the process, for the AdamW / hash pipeline.  The whole
// enqueue sequence of a call runs under one lock, so concurrent callers on
// one device never interleave their event records.
struct SideStream {
  hipStream_t stream[2] = {nullptr, nullptr};
  std::vector<hipEvent_t> events;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mutex;
SideStream g_side[kMaxDevices];

hipError_t side_stream(int device, size_t nevents, SideStream** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  SideStream& r = g_side[device];
  for (hipStream_t& st : r.stream) {
    if (st == nullptr) {
      const hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
      if (e != hipSuccess) return e;
    }
  }
  while (r.events.size() < nevents) {
    hipEvent_t ev;
    const hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    r.events.push_back(ev);
  }
  *out = &r;
  return hipSuccess;
}

constexpr int64_t kLeafWords = 1024;            // a 4096-byte hash leaf
// The largest word count the hash accepts: its byte count, and every level's
// digest bytes, stay far inside int64 (2^60 words = 4 EiB).
constexpr int64_t kMaxHashWords = int64_t(1) << 60;
// Pipelined form: 2^26 elements per chunk, 196,608 leaves per hash launch
// (768 workgroups), the fastest of 2^23 .. 2^28 measured on the optimizer
// workload.
constexpr int64_t kDefaultChunk = int64_t(1) << 26;

}  // namespace

int repro_adamw_hash(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2, float eps,
                     float weight_decay, int64_t step, void* workspace, int64_t ws_bytes, uint8_t* digest_out,
                     int64_t chunk, void* stream) {
  if (n < 0 || step < 1 || workspace == nullptr || digest_out == nullptr) return REPRO_EINVAL;
  if (n > kMaxHashWords / 3) return REPRO_EINVAL;
  if (chunk > 0 && chunk % kLeafWords != 0) return REPRO_EINVAL;
  if (n > 0 && (state == nullptr || grad == nullptr)) return REPRO_EINVAL;
  if (n > 0 && (!aligned4(state) || !aligned4(grad))) return REPRO_EALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0 || (reinterpret_cast<uintptr_t>(digest_out) & 15u) != 0)
    return REPRO_EALIGN;
  repro::HashPlan plan;
  repro::plan_state_hash(3 * n, &plan);
  if (ws_bytes < plan.total_bytes) return REPRO_ESPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const hipStream_t main = static_cast<hipStream_t>(stream);
  const AdamwScalars s = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step);
  const bool al16 = ((reinterpret_cast<uintptr_t>(state) | reinterpret_cast<uintptr_t>(grad)) & 15u) == 0;
  if (chunk == 0 && n > 0 && n % kLeafWords == 0 && al16)
    return status_of(repro::launch_adamw_hash_fused(state, grad, n, s, ws, plan, digest_out, main));
  if (chunk == 0) chunk = kDefaultChunk;
  // Without whole leaves per region (or asked not to), the two run in turn.
  if (chunk < 0 || n % kLeafWords != 0 || n <= chunk) {
    if (n > 0) {
      const hipError_t e = repro::launch_adamw(state, grad, n, s, 0, main);
      if (e != hipSuccess) return status_of(e);
    }
    return status_of(repro::launch_state_hash(state, 3 * n, ws, plan, digest_out, main));
  }
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return status_of(e);
  const int64_t nchunks = (n + chunk - 1) / chunk;
  std::lock_guard<std::mutex> lock(g_side_mutex);
  SideStream* side = nullptr;
  e = side_stream(device, (size_t)nchunks + 3, &side);
  if (e != hipSuccess) return status_of(e);
  // Fork: the side streams start after everything already on the caller's.
  if ((e = hipEventRecord(side->events[0], main)) != hipSuccess) return status_of(e);
  for (hipStream_t st : side->stream)
    if ((e = hipStreamWaitEvent(st, side->events[0], 0)) != hipSuccess) return status_of(e);
  const int64_t leaves_per_region = n / kLeafWords;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t first = c * chunk;
    const int64_t count = n - first < chunk ? n - first : chunk;
    e = repro::launch_adamw_ptrs(state + first, state + n + first, state + 2 * n + first, grad + first, count, s, 0,
                                 main);
    if (e != hipSuccess) return status_of(e);
    hipEvent_t done = side->events[(size_t)c + 1];
    if ((e = hipEventRecord(done, main)) != hipSuccess) return status_of(e);
    // This chunk's leaves in w, m and v, in one launch; chunks alternate
    // between the two side streams so one launch's tail overlaps the next.
    hipStream_t hs = side->stream[c & 1];
    if ((e = hipStreamWaitEvent(hs, done, 0)) != hipSuccess) return status_of(e);
    e = repro::launch_hash_leaves(state, 3 * n, ws, plan, first / kLeafWords, count / kLeafWords, leaves_per_region,
                                  3, hs);
    if (e != hipSuccess) return status_of(e);
  }
  // Join, then the levels above the leaves on the caller's stream.
  for (int k = 0; k < 2; ++k) {
    hipEvent_t joined = side->events[(size_t)nchunks + 1 + k];
    if ((e = hipEventRecord(joined, side->stream[k])) != hipSuccess) return status_of(e);
    if ((e = hipStreamWaitEvent(main, joined, 0)) != hipSuccess) return status_of(e);
  }
  return status_of(repro::launch_hash_upper(ws, plan, digest_out, main));
}

namespace {

// Workspace of repro_adamw_hash_noalloc: one array per device, placed by the
// code-object loader, so the call needs no allocation of any kind.  In host
// code the name `scratch` is only a stand-in for the symbol; the device
// address comes from hipGetSymbolAddress, once per device, and only that
// address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[REPRO_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's `scratch`, looked up on the
// first call made on that device.
hipError_t scratch_address(void** out) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace

int repro_adamw_hash_noalloc(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2,
                             float eps, float weight_decay, int64_t step, uint8_t* digest_out, void* stream) {
  if (n < 0 || step < 1 || digest_out == nullptr) return REPRO_EINVAL;
  if (n > 0 && (state == nullptr || grad == nullptr)) return REPRO_EINVAL;
  if (n > 0 && (!aligned4(state) || !aligned4(grad))) return REPRO_EALIGN;
  if ((reinterpret_cast<uintptr_t>(digest_out) & 15u) != 0) return REPRO_EALIGN;
  if (n > INT64_MAX / 3) return REPRO_ESPACE;
  repro::HashPlan plan;
  repro::plan_state_hash(3 * n, &plan);
  if (plan.total_bytes > REPRO_NOALLOC_SCRATCH_BYTES) return REPRO_ESPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return status_of(e);
  const hipStream_t main = static_cast<hipStream_t>(stream);
  const AdamwScalars s = adamw_scalars(lr, beta1, beta2, eps, weight_decay, step);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  const bool al16 = ((reinterpret_cast<uintptr_t>(state) | reinterpret_cast<uintptr_t>(grad)) & 15u) == 0;
  if (n > 0 && n % kLeafWords == 0 && al16)
    return status_of(repro::launch_adamw_hash_fused(state, grad, n, s, wsb, plan, digest_out, main));
  // Otherwise the update and then the hash, both on the caller's stream.
  if (n > 0) {
    const hipError_t e2 = repro::launch_adamw(state, grad, n, s, 0, main);
    if (e2 != hipSuccess) return status_of(e2);
  }
  return status_of(repro::launch_state_hash(state, 3 * n, wsb, plan, digest_out, main));
}

int64_t repro_state_hash_workspace_bytes(int64_t n_words) {
  if (n_words < 0 || n_words > kMaxHashWords) return REPRO_EINVAL;
  repro::HashPlan plan;
  repro::plan_state_hash(n_words, &plan);
  return plan.total_bytes;
}

int repro_state_hash(const float* words, int64_t n_words, void* workspace, int64_t ws_bytes, uint8_t* digest_out,
                     void* stream) {
  if (n_words < 0 || n_words > kMaxHashWords || workspace == nullptr || digest_out == nullptr) return REPRO_EINVAL;
  if (n_words > 0 && words == nullptr) return REPRO_EINVAL;
  if (n_words > 0 && !aligned4(words)) return REPRO_EALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0 || (reinterpret_cast<uintptr_t>(digest_out) & 15u) != 0)
    return REPRO_EALIGN;
  repro::HashPlan plan;
  repro::plan_state_hash(n_words, &plan);
  if (ws_bytes < plan.total_bytes) return REPRO_ESPACE;
  return status_of(repro::launch_state_hash(words, n_words, static_cast<uint8_t*>(workspace), plan, digest_out,
                                            static_cast<hipStream_t>(stream)));
}

int repro_fp32_ops(int32_t op, const float* a, const float* b, float* out, int64_t n, void* stream) {
  if (op < 0 || op > 4 || n < 0) return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (a == nullptr || b == nullptr || out == nullptr) return REPRO_EINVAL;
  if (!aligned4(a) || !aligned4(b) || !aligned4(out)) return REPRO_EALIGN;
  return status_of(repro::launch_fp32_ops(op, a, b, out, n, static_cast<hipStream_t>(stream)));
}

int64_t repro_grad_norm_workspace_bytes(int64_t n) {
  if (n < 0) return REPRO_EINVAL;
  repro::NormPlan plan;
  repro::plan_grad_norm(n, &plan);
  return plan.total_bytes;
}

namespace {

int check_grad(const void* grad, int32_t dtype, int64_t n, void* workspace, int64_t ws_bytes,
               repro::NormPlan* plan) {
  if (n < 0 || (dtype != REPRO_GRAD_F32 && dtype != REPRO_GRAD_BF16) || workspace == nullptr) return REPRO_EINVAL;
  if (n > 0 && grad == nullptr) return REPRO_EINVAL;
  if (n > 0 && (reinterpret_cast<uintptr_t>(grad) & (dtype == REPRO_GRAD_BF16 ? 1u : 3u)) != 0) return REPRO_EALIGN;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return REPRO_EALIGN;
  repro::plan_grad_norm(n, plan);
  if (ws_bytes < plan->total_bytes) return REPRO_ESPACE;
  return REPRO_OK;
}

}  // namespace

int repro_grad_norm(const void* grad, int32_t grad_dtype, int64_t n, void* workspace, int64_t ws_bytes,
                    float* out2, void* stream) {
  repro::NormPlan plan;
  const int st = check_grad(grad, grad_dtype, n, workspace, ws_bytes, &plan);
  if (st != REPRO_OK) return st;
  if (out2 == nullptr) return REPRO_EINVAL;
  if (!aligned4(out2)) return REPRO_EALIGN;
  const repro::StepRule rule = {0.0f, 0.0f, 0.0f, 0.0f, 0};
  return status_of(repro::launch_grad_norm(grad, grad_dtype, n, static_cast<uint8_t*>(workspace), plan, out2,
                                           nullptr, rule, static_cast<hipStream_t>(stream)));
}

int repro_adamw_bf16_step(uint16_t* w, float* m, float* v, const void* grad, int32_t grad_dtype, int64_t n,
                          float lr, float beta1, float beta2, float eps, float weight_decay, float max_norm,
                          float spike_threshold, int32_t skip_steps, void* workspace, int64_t ws_bytes,
                          repro_step_state* state, void* stream) {
  repro::NormPlan plan;
  const int st = check_grad(grad, grad_dtype, n, workspace, ws_bytes, &plan);
  if (st != REPRO_OK) return st;
  if (state == nullptr || skip_steps < 0) return REPRO_EINVAL;
  if ((reinterpret_cast<uintptr_t>(state) & 7u) != 0) return REPRO_EALIGN;
  if (n > 0) {
    if (w == nullptr || m == nullptr || v == nullptr) return REPRO_EINVAL;
    if ((reinterpret_cast<uintptr_t>(w) & 1u) != 0 || !aligned4(m) || !aligned4(v)) return REPRO_EALIGN;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const repro::StepRule rule = {beta1, beta2, max_norm, spike_threshold, skip_steps};
  hipError_t e = repro::launch_grad_norm(grad, grad_dtype, n, static_cast<uint8_t*>(workspace), plan, nullptr, state,
                                         rule, s);
  if (e != hipSuccess) return status_of(e);
  if (n == 0) return REPRO_OK;
  return status_of(repro::launch_adamw_bf16(w, m, v, grad, grad_dtype, n, static_cast<const uint8_t*>(workspace), lr,
                                            beta1, beta2, eps, weight_decay, s));
}

int repro_fp32_fma(const float* a, const float* b, const float* c, float* out, int64_t n, int32_t unit,
                   void* stream) {
  if (unit < 0 || unit > 3 || n < 0) return REPRO_EINVAL;
  if (n == 0) return REPRO_OK;
  if (a == nullptr || b == nullptr || c == nullptr || out == nullptr) return REPRO_EINVAL;
  if (!aligned4(a) || !aligned4(b) || !aligned4(c) || !aligned4(out)) return REPRO_EALIGN;
  return status_of(repro::launch_fp32_fma(unit, a, b, c, out, n, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
