// Internal interface between the C-ABI front end (api.cpp) and the kernel
// translation units.  Every launcher enqueues on `stream` and returns the
// hipError_t of the launch; argument checking is done by the front end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "repro.h"

namespace repro {

struct ReplicaPtrs {
  const float* p[REPRO_MAX_REPLICAS];
};

// Algorithm 1 replay: the N * accum gradient buffers in mesh order.
struct ReplayPtrs {
  const float* p[REPRO_MAX_REPLAY_BUFFERS];
};

// Streaming TreeFold: one device buffer per fold level.
constexpr int kFoldSlots = REPRO_FOLD_SLOTS;
struct FoldSlotPtrs {
  float* p[kFoldSlots];
};

// Host-prepared AdamW scalars (binary32, computed under the contract).
struct AdamwScalars {
  float lr, beta1, beta2, eps, wd;
  float c1, c2, r1, r2;
};

// elementwise.hip
hipError_t launch_tree_reduce(const ReplicaPtrs& reps, int R, int64_t n, float* out, int average, float rR,
                              int variant, hipStream_t stream);
hipError_t launch_adamw(float* state, const float* grad, int64_t n, const AdamwScalars& s, int variant,
                        hipStream_t stream);
// The same update on `count` elements of separate w, m, v, g arrays.
hipError_t launch_adamw_ptrs(float* w, float* m, float* v, const float* grad, int64_t count, const AdamwScalars& s,
                             int variant, hipStream_t stream);
hipError_t launch_fp32_ops(int op, const float* a, const float* b, float* out, int64_t n, hipStream_t stream);

// replay.hip
hipError_t launch_replay(const ReplayPtrs& a, int nbuf, int dp_replicate, int dp_shard, int accum, float r_accum,
                         float r_shard, float r_rep, int64_t n, float* out, hipStream_t stream);
hipError_t launch_fold_push(const FoldSlotPtrs& sl, int t, const float* part, int64_t n, hipStream_t stream);
hipError_t launch_fold_result(const FoldSlotPtrs& sl, int pushed, int average, float r, float* out, int64_t n,
                              hipStream_t stream);

// gemm.hip
hipError_t launch_gemm(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                       const float* B, int64_t ldb, float* C, int64_t ldc, int variant, bool fused,
                       hipStream_t stream);

// optimizer.hip
struct OptHeader {  // first bytes of the grad-norm / optimizer workspace
  float norm;       // the pre-clip global norm
  float sumsq;      // the fold of the squares
  int apply;        // 1: the step applies its update
  float coef;       // clip coefficient (1: no clip)
  float c1, c2, r1, r2;
};
constexpr int64_t kOptHeaderBytes = 256;
struct NormPlan {
  static constexpr int kMaxPasses = 8;
  int passes;
  int64_t len[kMaxPasses];         // input length of each pass
  int64_t out_offset[kMaxPasses];  // workspace offset of its block sums (-1: the header)
  int64_t total_bytes;
};
struct StepRule {
  float beta1, beta2, max_norm, spike_threshold;
  int skip_steps;
};
void plan_grad_norm(int64_t n, NormPlan* plan);
hipError_t launch_grad_norm(const void* g, int dtype, int64_t n, uint8_t* ws, const NormPlan& plan, float* out2,
                            repro_step_state* st, const StepRule& rule, hipStream_t stream);
hipError_t launch_adamw_bf16(uint16_t* w, float* m, float* v, const void* g, int dtype, int64_t n, const uint8_t* ws,
                             float lr, float beta1, float beta2, float eps, float wd, hipStream_t stream);

// fused.hip
hipError_t launch_fp32_fma(int unit, const float* a, const float* b, const float* c, float* out, int64_t n,
                           hipStream_t stream);

// state_hash.hip
struct HashPlan {
  static constexpr int kMaxLevels = 64;
  int levels;                       // number of levels, leaves included
  int64_t count[kMaxLevels];        // nodes per level
  int64_t offset[kMaxLevels];       // byte offset of each level's digests in the workspace
  int64_t total_bytes;              // workspace bytes needed
};
void plan_state_hash(int64_t n_words, HashPlan* plan);
// Level 0 only: `ranges` runs of `count` leaves at first + r * stride; then
// the levels above.
hipError_t launch_hash_leaves(const float* words, int64_t n_words, uint8_t* workspace, const HashPlan& plan,
                              int64_t first, int64_t count, int64_t stride, int ranges, hipStream_t stream);
hipError_t launch_hash_upper(uint8_t* workspace, const HashPlan& plan, uint8_t* digest_out, hipStream_t stream);
// AdamW on [w | m | v] and the whole state hash, the update and the leaf
// level in one kernel (n a multiple of 1024, state and grad 16-byte aligned).
hipError_t launch_adamw_hash_fused(float* state, const float* grad, int64_t n, const AdamwScalars& s, uint8_t* ws,
                                   const HashPlan& plan, uint8_t* digest_out, hipStream_t stream);
hipError_t launch_state_hash(const float* words, int64_t n_words, uint8_t* workspace, const HashPlan& plan,
                             uint8_t* digest_out, hipStream_t stream);

}  // namespace repro
