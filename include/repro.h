/*
 * repro.h - C ABI of librepro.so: bitwise-reproducible training-step
 * operations for AMD Instinct MI355X (gfx950).
 *
 * The operations are the order-fixed "reproducible operations" of
 * "OPEN-1B: A Fully Auditable Training Run" (Gensyn):
 *   - section 2 and 2.1 with Table 1: results are equal bit for bit, with one
 *     fixed reduction order, multiply and add unfused, and subnormal
 *     operands and results flushed to zero;
 *   - Appendix A.1 with Algorithm 2 (TreeFold) and Appendix A.3 (an average is
 *     a multiply by a host-computed reciprocal);
 *   - section 3.2 "Optimizer" and "Optimizer-state precision" (fused FP32
 *     AdamW with decoupled weight decay);
 *   - Appendix B and Figure 11 (a BLAKE2b state hash per step).
 *
 * Numeric contract shared by every call: IEEE 754 binary32, round to
 * nearest even, no fused multiply-add.  Subnormals are flushed the way the
 * processor path's FTZ and DAZ modes do it (section 2.1 "Subnormals"), with
 * the x86 definition of those modes: a subnormal operand reads as a zero of
 * the same sign, and a result that is tiny - below 2^-126 once rounded to 24
 * significant bits with an unbounded exponent - becomes a zero of the same
 * sign.  Division and square root are correctly rounded.  Inputs are assumed
 * finite.
 *
 * Determinism promise: output bits depend only on the input bits and the
 * arguments, never on the stream, the launch configuration (the *_variant
 * entry points select alternative launch shapes that must give the same
 * bits), the device, or the process.
 *
 * Conventions for every call:
 *   - Pointers named "device" point to device memory (a hipMalloc'd
 *     allocation, e.g. a torch tensor on a ROCm device) and must be aligned
 *     to 4 bytes.  16-byte alignment enables the vectorised kernels; other
 *     alignments take a slower path with identical results.
 *   - The caller owns every buffer.  The library allocates no device memory.
 *     Its only global state is a pair of streams and a pool of events per
 *     device, created by the first repro_adamw_hash call with chunk > 0 and
 *     kept until the process ends, and the workspace array of
 *     repro_adamw_hash_noalloc (one per device, see there).  Calls are
 *     thread-safe, except that repro_adamw_hash_noalloc calls overlapping on
 *     one device share that array.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and returns without waiting.
 *   - Return value: REPRO_OK (0) or a negative REPRO_E* code.  On an error
 *     nothing has been enqueued, except REPRO_EDEVICE, which reports a HIP
 *     launch failure (hipGetLastError) after the launch.
 */
#ifndef REPRO_H
#define REPRO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define REPRO_OK 0
#define REPRO_EINVAL -1 /* null pointer, negative size, bad flag, R out of range, ld too small, step < 1 */
#define REPRO_EALIGN -2 /* a pointer is not aligned as the call requires (4 bytes unless stated) */
#define REPRO_EDEVICE -3 /* HIP launch or runtime error */
#define REPRO_ESPACE -4 /* workspace too small */

#define REPRO_MAX_REPLICAS 64
#define REPRO_MAX_REPLAY_BUFFERS 384
#define REPRO_FOLD_SLOTS 7

/* "repro-spec-1": names the orders, the constants and the hash parameters
 * below.  A change to any of them changes this string. */
const char* repro_spec_version(void);

/* Static description of a status code. */
const char* repro_strerror(int status);

/*
 * repro_gemm: C = op(A) * op(B), binary32, row-major.
 *
 * Paper section 2.1 "Reduction order" (one fixed order for every sum in a
 * matrix multiply) and "Fused multiply-add" (unfused); section 6 item 1.
 * Each C[i][j] is one serial chain: acc = +0, then for k = 0, 1, ..., K-1
 * in ascending order acc = fl(acc + fl(opA[i][k] * opB[k][j])).  The kernel
 * tiles only over outputs and never splits k.
 *
 *   op(A) is M x K: A[i*lda + k], or A[k*lda + i] when trans_a != 0
 *   op(B) is K x N: B[k*ldb + j], or B[j*ldb + k] when trans_b != 0
 *   C[i*ldc + j], M x N.
 * Requirements: M, N, K >= 0; ldc >= N; when K > 0, lda >= (trans_a ? M : K)
 * and ldb >= (trans_b ? K : N).  A, B, C are device pointers; C must not
 * overlap A or B.  M == 0 or N == 0: nothing to do.  K == 0: C = +0.
 */
int repro_gemm(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
               const float* B, int64_t ldb, float* C, int64_t ldc, void* stream);

/* As repro_gemm with an explicit kernel variant.  0 is the default, the
 * kernel of variant 3.  3 forms each product fl(a*b) on the matrix cores
 * (v_mfma_f32_32x32x1_2b_f32 with K = 1 and C = -0, one product per output
 * element, nothing summed inside) and adds it into the output's chain on the
 * VALU (128x128 tiles).  4 multiplies and adds on the VALU (256x128 tiles
 * when the output holds at least 512 of them, else 128x128); 1 does the same
 * with scalar global loads and 128x128 tiles; 2 with 64x64 tiles.  All
 * variants return the same bits; they exist to test that claim. */
int repro_gemm_variant(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A,
                       int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc, int32_t variant,
                       void* stream);

/*
 * repro_gemm_fma: the same GEMM under a declared fused multiply-add
 * convention, which the pages do not use (paper section 2.1 "Fused
 * multiply-add" keeps multiply and add unfused on every backend).  It is
 * for callers that declare this convention for their whole run; its results
 * differ from repro_gemm's.
 *
 * Each C[i][j] is one serial chain over k = 0, 1, ..., K-1 ascending:
 * acc = +0, then acc = fma(opA[i][k], opB[k][j], acc), where fma(a, b, c) is
 * a*b + c rounded once to binary32 (nearest-even) under the contract's
 * subnormal rule: subnormal operands read as zeros of the same sign, and a
 * result below 2^-126 after rounding to 24 bits (unbounded exponent) becomes
 * a zero of the same sign.  Arguments, layout and errors as repro_gemm.
 *
 *   variant 0: matrix cores.  v_mfma_f32_32x32x1_2b_f32 with K = 1 takes the
 *              chain value as its C operand, which is exactly one fused step
 *              per output; consecutive instructions walk k in order.
 *   variant 1: VALU, one v_fma_f32 per step (the unfused default's tiles:
 *              256x128 for outputs with at least 512 of them, else 128x128).
 * Both variants return the same bits.
 */
int repro_gemm_fma(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                   const float* B, int64_t ldb, float* C, int64_t ldc, int32_t variant, void* stream);

/*
 * repro_tree_reduce: out[i] = Fold(x_0[i], ..., x_{R-1}[i]) (times fl(1/R)).
 *
 * Paper Appendix A.1 with Algorithm 2: TreeFold, the binary-carry fold that
 * reproduces the recursive-doubling all-reduce order over replicas.  Push
 * combines equal-size blocks with the lower replicas on the left; Result
 * starts from the smallest remaining block and adds the larger ones in turn,
 * so for R = 8 the sum is ((x0+x1)+(x2+x3))+((x4+x5)+(x6+x7)) and for
 * R = 7 it is (x6+(x4+x5))+((x0+x1)+(x2+x3)).  Appendix A.3: when average
 * is nonzero the fold is multiplied by rR = fl(1/R), a binary32 reciprocal
 * computed on the host; it is never a division.
 *
 *   replicas: HOST array of R device pointers, each to n floats (replica
 *             gradient buffers in replica order 0..R-1).  The array itself
 *             is read during the call only.
 *   R:        1 <= R <= REPRO_MAX_REPLICAS.
 *   out:      device pointer to n floats.  It may be one of the replicas
 *             (each element is read before it is written) but must not
 *             partially overlap any of them.
 *   average:  0 = plain fold, nonzero = fold * fl(1/R).
 * n == 0: nothing to do.
 */
int repro_tree_reduce(const float* const* replicas, int32_t R, int64_t n, float* out, int32_t average,
                      void* stream);

/* Variant 0 default (16-byte vectors, one-wave workgroups); 1 scalar elements;
 * 2 16-byte vectors, 64 threads and a grid-stride loop over a small grid. */
int repro_tree_reduce_variant(const float* const* replicas, int32_t R, int64_t n, float* out,
                              int32_t average, int32_t variant, void* stream);

/*
 * repro_replay_reduce: the audit replay of one step's gradient reduction.
 *
 * Paper section 6, Algorithm 1, with Appendix A.1 (TreeFold over replicas),
 * A.2 (ascending-shard sum) and A.3 (every average a multiply by a
 * host-computed reciprocal).  N = dp_replicate * dp_shard virtual ranks in
 * mesh order r = rep * dp_shard + shard; rank r has `accum` microbatch
 * gradients, grads[r * accum + k].  Per element:
 *   g_r = +0, then g_r = g_r + grad[r][k] * fl(1/accum) for k = 0..accum-1;
 *   inner = g_r for shard 0, inner = inner + g_r for shards 1..dp_shard-1;
 *   at the replica's last shard: Push(inner * fl(1/dp_shard));
 *   out = Result() * fl(1/dp_replicate)   (TreeFold as in repro_tree_reduce).
 *
 *   grads: HOST array of dp_replicate * dp_shard * accum device pointers,
 *          each to n floats (at most REPRO_MAX_REPLAY_BUFFERS in all).
 *   dp_replicate: 1..REPRO_MAX_REPLICAS; dp_shard, accum: >= 1.
 *   out:   device pointer to n floats; may equal one of the buffers.
 * n == 0: nothing to do.
 */
int repro_replay_reduce(const float* const* grads, int32_t dp_replicate, int32_t dp_shard, int32_t accum,
                        int64_t n, float* out, void* stream);

/*
 * repro_fold_push / repro_fold_result: TreeFold (Appendix A.1, Algorithm 2)
 * as a streaming interface for partials that arrive one at a time, holding
 * at most floor(log2 R) + 1 partials ("at most 4" for R = 8).
 *
 *   slots:  HOST array of REPRO_FOLD_SLOTS device buffers of n floats, owned
 *           by the caller; slots[L] holds the fold's entry of level L, which
 *           exists exactly when bit L of `pushed` is set.  Only slots that
 *           the call reads or writes need to be valid pointers.
 *   pushed: the number of partials pushed before this call (the caller
 *           counts); push accepts 0..126, result 1..127.
 * repro_fold_push adds `part` to the occupied levels 0, 1, ... while their
 * bits are set (the earlier, lower block on the left) and stores the sum in
 * the first free level.  `part` may be that free slot.
 * repro_fold_result writes the lowest occupied level plus the others in
 * ascending level order to `out`, times fl(1/divisor) when divisor > 0.
 */
int repro_fold_push(float* const* slots, int32_t pushed, const float* part, int64_t n, void* stream);
int repro_fold_result(float* const* slots, int32_t pushed, int64_t n, float* out, int32_t divisor, void* stream);

/*
 * repro_adamw: one fused AdamW step, in place, on the flat binary32 state.
 *
 * Paper section 3.2 "Optimizer" (AdamW, decoupled weight decay, a
 * bitwise-reproducible fused kernel) and "Optimizer-state precision" (FP32
 * moments); the checkpoint page's file format gives the flat [w | m | v]
 * layout.  Host scalars (binary32, same contract): c1 = 1 - beta1,
 * c2 = 1 - beta2, p = beta^step by step-1 serial multiplies, r1 = 1/(1 - p1),
 * r2 = 1/(1 - p2) (Appendix A.3's reciprocal rule applied to the bias
 * corrections).  Per element, in this order, each step one rounding:
 *   m1 = beta1*m   m2 = c1*g   m' = m1 + m2
 *   q = g*g        v1 = beta2*v  v2 = c2*q  v' = v1 + v2
 *   mh = m'*r1     vh = v'*r2
 *   s = sqrt(vh)   d = s + eps   u = mh / d
 *   y = wd*w       z = u + y     t = lr*z   w' = w - t
 *
 *   state: device pointer to 3n floats: w = state[0..n), m = state[n..2n),
 *          v = state[2n..3n).  Updated in place (w', m', v').
 *   grad:  device pointer to n floats; must not overlap state.
 *   step:  the step being taken, >= 1.
 * n == 0: nothing to do.
 */
int repro_adamw(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2, float eps,
                float weight_decay, int64_t step, void* stream);

/* Variant 0 default (16-byte vectors); 1 scalar elements. */
int repro_adamw_variant(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2,
                        float eps, float weight_decay, int64_t step, int32_t variant, void* stream);

/*
 * BF16-parameter optimizer step with the global-norm clip and the spike rule.
 *
 * Paper section 3.1 (parameters held in BF16, FP32 gradient reduction),
 * section 3.2 "Optimizer" (AdamW; gradients clipped to a global l2 norm of
 * 1.0) and "Optimizer-state precision" (the fused step widens the BF16
 * parameter and gradient to FP32, updates in FP32 with FP32 moments, rounds
 * the parameter to BF16 once), section 3.4.2 (five optimizer steps are
 * skipped when the pre-clip gradient norm exceeds 5).
 *
 * The pre-clip norm: q_i = g_i * g_i in binary32 (bf16 gradients widened
 * first), S = TreeFold(q_0, ..., q_{n-1}) in index order (Appendix A.1's
 * fold applied to scalars: equal blocks combined as in binary counting,
 * Result from the smallest block upward), norm = sqrt(S) correctly rounded.
 *
 * One step, all in binary32 under the contract:
 *   spike rule (spike_threshold > 0): norm > spike_threshold sets
 *     skip_left = skip_steps, so this step and the next skip_steps - 1 are
 *     skipped (a spike inside the window starts it again);
 *   skipped (skip_left > 0, then decremented): w, m, v and step unchanged;
 *   clip (max_norm > 0): c = max_norm / (norm + 1e-6); when c < 1 every
 *     gradient element is multiplied by c (one product each);
 *   applied: t = step + 1, beta^t carried as one more serial multiply of
 *     beta_pow (beta itself at t = 1), c1, c2, r1 = 1/(1 - beta1^t),
 *     r2 = 1/(1 - beta2^t), then per element the sixteen operations of
 *     repro_adamw on (widen(w), m, v, g), and w' rounded to bf16 (nearest,
 *     ties to even) once.
 */
typedef struct repro_step_state {
  int64_t step;      /* updates applied so far */
  int32_t skip_left; /* steps still to skip */
  int32_t applied;   /* 1 if the last step applied its update */
  float beta1_pow;   /* beta1^step (not read while step == 0) */
  float beta2_pow;   /* beta2^step */
  float grad_norm;   /* the last step's pre-clip norm */
  float clip_coef;   /* the coefficient applied to its gradient (1: none) */
} repro_step_state;  /* 32 bytes; all zero = no step taken yet */

#define REPRO_GRAD_F32 0
#define REPRO_GRAD_BF16 1

/* Workspace bytes for n gradient elements (block sums of the norm's fold
 * and the step's scalars); at least 256. */
int64_t repro_grad_norm_workspace_bytes(int64_t n);

/*
 * repro_grad_norm: out2[0] = the pre-clip norm above, out2[1] = S.
 *   grad:      device pointer to n elements of grad_dtype (REPRO_GRAD_F32,
 *              4-byte aligned, or REPRO_GRAD_BF16, 2-byte aligned).
 *   workspace: device memory, 256-byte aligned, of at least
 *              repro_grad_norm_workspace_bytes(n) bytes (REPRO_ESPACE
 *              otherwise).
 *   out2:      device pointer to 2 floats, written last.
 * n == 0: norm = S = 0.  Asynchronous on the stream.
 */
int repro_grad_norm(const void* grad, int32_t grad_dtype, int64_t n, void* workspace, int64_t ws_bytes,
                    float* out2, void* stream);

/*
 * repro_adamw_bf16_step: one optimizer step, in place and asynchronous.
 *   w:     device pointer to n bf16 parameters (uint16 bit patterns).
 *   m, v:  device pointers to n floats each (FP32 moments).
 *   grad:  as repro_grad_norm; must not overlap w, m or v.
 *   max_norm <= 0 disables the clip, spike_threshold <= 0 the spike rule;
 *   skip_steps >= 0.
 *   workspace: as repro_grad_norm.
 *   state: device pointer to the caller's repro_step_state (8-byte
 *          aligned), read and updated by the step; zero it before the first.
 * The step count, the skip window and the beta powers live in `state`, so
 * consecutive calls need no host synchronisation.  Calls that share a
 * workspace or a state must be ordered on one stream.
 */
int repro_adamw_bf16_step(uint16_t* w, float* m, float* v, const void* grad, int32_t grad_dtype, int64_t n,
                          float lr, float beta1, float beta2, float eps, float weight_decay, float max_norm,
                          float spike_threshold, int32_t skip_steps, void* workspace, int64_t ws_bytes,
                          repro_step_state* state, void* stream);

/*
 * repro_state_hash: 32-byte BLAKE2b tree digest of n_words binary32 words.
 *
 * Paper Appendix B (a canonical per-step state hash) and Figure 11 (the hash
 * is BLAKE2b); section 3.2 (state hashed in FP32).  BLAKE2b as RFC 7693, in
 * the tree mode of the BLAKE2 paper (section 2.10) with digest length 32,
 * fanout 16, depth 255, leaf length 4096, inner length 32 and
 * personalisation "repro_state_v1" (zero-padded to 16 bytes), over the
 * little-endian bytes of the words:
 *   level 0: leaves of 4096 bytes (the last may be shorter; no words = one
 *            empty leaf), leaf i at node offset i, node depth 0;
 *   level d >= 1: node j hashes the concatenated digests of children
 *            16j .. 16j+15 of level d-1, node offset j, node depth d;
 *   the last node of every level carries the last-node flag; levels are
 *   added until one node remains, always at least one above the leaves.
 * The root digest is the state hash.  Hash [w | m | v] by passing
 * state and 3n.
 *
 *   words:      device pointer to n_words floats (0 <= n_words <= 2^60;
 *               larger counts return REPRO_EINVAL, as does
 *               repro_state_hash_workspace_bytes for them).
 *   workspace:  device memory of at least
 *               repro_state_hash_workspace_bytes(n_words) bytes, 16-byte
 *               aligned, used for the digests of every level.
 *   digest_out: device pointer to 32 bytes, written last.
 */
int64_t repro_state_hash_workspace_bytes(int64_t n_words);
int repro_state_hash(const float* words, int64_t n_words, void* workspace, int64_t ws_bytes,
                     uint8_t* digest_out, void* stream);

/*
 * repro_adamw_hash: repro_adamw on the flat state, then repro_state_hash of
 * the updated [w | m | v] (3n words), with the same results bit for bit.
 *
 * Paper section 3.2 (the fused step) and Appendix B with Figure 11 (the
 * per-step state hash, whose move from the host onto the device the pages
 * name as their next step).  The update is bound by memory traffic and the
 * hash by integer arithmetic, so they are not run one after the other:
 *   chunk == 0 (default): one kernel updates each 128-byte block of every
 *          leaf and hashes it from on-chip memory right away, so the
 *          updated state is written once and never read back; the levels
 *          above the leaves follow.  Needs n a multiple of 1024 (so no leaf
 *          straddles w, m and v) and 16-byte aligned state and grad;
 *          otherwise the call proceeds as for chunk == 2^26.
 *   chunk > 0: a multiple of 1024; the update runs in chunks of `chunk`
 *          elements on the caller's stream, and as each chunk completes the
 *          leaves it covers in w, m and v are hashed on a second stream of
 *          the library's (when n is not a multiple of 1024, or n <= chunk,
 *          the two run in turn);
 *   chunk < 0: the update, then the hash, both on the caller's stream.
 *
 *   state, grad, n, lr ... step: as repro_adamw (n <= 2^60 / 3).
 *   workspace, ws_bytes: as repro_state_hash for 3n words.
 *   digest_out: device pointer to 32 bytes (16-byte aligned).
 * Asynchronous: the caller's stream is ordered after all of the work.  For
 * chunk > 0 the library's second streams and their events are created on
 * the first such call on a device and live until the process ends; each
 * call enqueues under a lock.
 */
int repro_adamw_hash(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2, float eps,
                     float weight_decay, int64_t step, void* workspace, int64_t ws_bytes, uint8_t* digest_out,
                     int64_t chunk, void* stream);

/*
 * repro_adamw_hash_noalloc: repro_adamw_hash (chunk == 0) for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, or harnesses that forbid allocation.  Same update, same
 * digest, bit for bit, with no workspace argument.
 *
 * The hash digests of every level live in a device array that the library
 * holds on each device it runs on (REPRO_NOALLOC_SCRATCH_BYTES, placed when
 * the library's code is loaded onto that device and kept until the process
 * ends); the call allocates nothing, frees nothing and creates no stream or
 * event.  Nothing in the array needs to start at zero: every digest slot is
 * written before it is read.  All calls on one device share that array, so
 * calls that overlap in time on one device (concurrent streams, or host
 * threads on different streams) race and must be serialised by the caller,
 * e.g. by using one stream.
 *
 *   state, grad, n, lr ... step: as repro_adamw.  With n a multiple of 1024
 *          and 16-byte aligned state and grad, one kernel updates and hashes
 *          the leaves; otherwise the update and then the hash run in turn on
 *          the caller's stream.
 *   digest_out: device pointer to 32 bytes (16-byte aligned).
 * REPRO_ESPACE when the hash of 3n words needs more than the array holds
 * (repro_state_hash_workspace_bytes(3n) > REPRO_NOALLOC_SCRATCH_BYTES, i.e.
 * n above about 1.34e9); nothing is enqueued then.  Asynchronous.
 */
#define REPRO_NOALLOC_SCRATCH_BYTES (128LL << 20)
int repro_adamw_hash_noalloc(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2,
                             float eps, float weight_decay, int64_t step, uint8_t* digest_out, void* stream);

/*
 * repro_fp32_ops: one contract operation per element, out[i] = a[i] op b[i],
 * in the same device arithmetic the kernels use (a diagnostic entry point for
 * directed tests of the flush rule, division and square root).
 *   op 0 add, 1 sub, 2 mul, 3 div, 4 sqrt (of a; b is read but ignored).
 * a, b, out: device pointers to n floats.
 */
int repro_fp32_ops(int32_t op, const float* a, const float* b, float* out, int64_t n, void* stream);

/*
 * repro_fp32_fma: out[i] = fma(a[i], b[i], c[i]) under the fused convention
 * of repro_gemm_fma, on one chosen unit: 0 = VALU v_fma_f32; 1, 2, 3 = the
 * matrix-core instructions with K = 1, v_mfma_f32_32x32x1_2b_f32,
 * v_mfma_f32_16x16x1_4b_f32 and v_mfma_f32_4x4x1_16b_f32 (each element
 * placed on the diagonal of a block, with c[i] as the C operand).  For
 * directed tests of the single step a fused chain repeats on each unit.
 * Device pointers of n floats; out may be the same pointer as a, b or c (no
 * partial overlap).
 */
int repro_fp32_fma(const float* a, const float* b, const float* c, float* out, int64_t n, int32_t unit,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* REPRO_H */
