/*
 * CPU oracle for the reproducible training-step operations.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the GPU library and is deliberately plain: one thread, literal loops, every
 * floating-point operation written out in the order the definition states.
 *
 * Source of every rule: "OPEN-1B: A Fully Auditable Training Run" (Gensyn).
 *   - Section 2 and 2.1 with Table 1: bit-for-bit equality, one fixed
 *     reduction order, unfused multiply then add, subnormals flushed to zero
 *     (FTZ on results, DAZ on inputs) everywhere.
 *   - Section 3.2 "Optimizer" and "Optimizer-state precision": fused AdamW,
 *     decoupled weight decay, FP32 moments, state hashed in FP32.
 *   - Section 6, Algorithm 1, and Appendix A.1-A.3 with Algorithm 2: the
 *     TreeFold order over replicas and averages as a multiply by a
 *     host-computed reciprocal.
 *   - Appendix B and Figure 11: the per-step state hash is BLAKE2b.
 * The checkpoint page ("grow a language model: checkpoints", section on the
 * file format) fixes the flat [w | m | v] order and beta2 = 0.999.
 * BLAKE2b itself follows RFC 7693 (Saarinen and Aumasson, 2015).
 * One declared alternative the pages do not use: a fused multiply-add GEMM
 * convention (oracle_fma, oracle_gemm_fma), for matrix-core chains.
 *
 * Floating-point model.  Section 2.1 has the processor path flush subnormals
 * by turning on its FTZ and DAZ modes.  On this x86-64 host those are the
 * MXCSR bits FTZ (15) and DAZ (6): every binary32 operation below runs on the
 * SSE unit with round-to-nearest-even, a subnormal operand read as a zero of
 * the same sign, and a result replaced by a zero of the same sign when it is
 * tiny, i.e. when its value rounded to 24 significant bits with an unbounded
 * exponent is below 2^-126 (Intel SDM vol. 1, "Numeric Underflow Exception"
 * and "Flush-To-Zero").  Build with -ffp-contract=off so no multiply and add
 * are ever fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <xmmintrin.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -5

/* ------------------------------------------------------------------------ */
/* The binary32 contract: SSE operations under FTZ and DAZ.                  */

typedef struct { unsigned int saved; } fpenv_t;

static fpenv_t enter_contract(void) {
    fpenv_t e;
    e.saved = _mm_getcsr();
    /* RNE (RC = 00), FTZ (bit 15) and DAZ (bit 6) on, all exceptions masked. */
    _mm_setcsr((e.saved & ~0x6000u) | 0x8000u | 0x0040u | 0x1F80u);
    return e;
}

static void leave_contract(fpenv_t e) { _mm_setcsr(e.saved); }

/* One binary32 operation each; the control register does the flushing.
 * (-frounding-math keeps the compiler from folding any of them at build
 * time, where the run-time mode would not apply.) */
static float f_add(float a, float b) { return a + b; }
static float f_sub(float a, float b) { return a - b; }
static float f_mul(float a, float b) { return a * b; }
static float f_div(float a, float b) { return a / b; }
static float f_sqrt(float a) { return sqrtf(a); }

/* Single contract operations, exported for the directed tests.
 * op: 0 add, 1 sub, 2 mul, 3 div, 4 sqrt (b ignored). */
int oracle_fp32_ops(int op, const float* a, const float* b, float* out, int64_t n) {
    if (n < 0 || op < 0 || op > 4) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    for (int64_t i = 0; i < n; ++i) {
        switch (op) {
        case 0: out[i] = f_add(a[i], b[i]); break;
        case 1: out[i] = f_sub(a[i], b[i]); break;
        case 2: out[i] = f_mul(a[i], b[i]); break;
        case 3: out[i] = f_div(a[i], b[i]); break;
        default: out[i] = f_sqrt(a[i]); break;
        }
    }
    leave_contract(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* GEMM: C = op(A) * op(B), row-major.  Section 2.1 "Reduction order" and
 * "Fused multiply-add": every C[i][j] is one chain over k = 0, 1, ..., K-1,
 * starting from +0, with each step acc <- fl(acc + fl(a_ik * b_kj)).
 * op(A)[i][k] is A[i*lda + k], or A[k*lda + i] when trans_a is set;
 * op(B)[k][j] is B[k*ldb + j], or B[j*ldb + k] when trans_b is set. */
int oracle_gemm(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                const float* A, int64_t lda, const float* B, int64_t ldb,
                float* C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return ORACLE_EINVAL;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (ldc < N) return ORACLE_EINVAL;
    if (K > 0) {
        if (lda < (trans_a ? M : K) || ldb < (trans_b ? K : N)) return ORACLE_EINVAL;
    }
    fpenv_t e = enter_contract();
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float a = trans_a ? A[k * lda + i] : A[i * lda + k];
                float b = trans_b ? B[j * ldb + k] : B[k * ldb + j];
                acc = f_add(acc, f_mul(a, b));
            }
            C[i * ldc + j] = acc;
        }
    }
    leave_contract(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* The fused multiply-add convention (a declared alternative: the pages keep
 * multiply and add unfused, section 2.1 "Fused multiply-add").
 *
 * fma(a, b, c) = fl(a*b + c), one rounding, under the same subnormal rule as
 * every other operation: a subnormal a, b or c reads as a zero of the same
 * sign; the exact a*b + c is rounded to 24 significant bits with an
 * unbounded exponent, and a result whose magnitude is then below 2^-126
 * becomes a zero of the same sign.
 *
 * Written from that definition without any fused instruction: a*b is exact
 * in binary64 (two 24-bit significands make at most 48 bits), the sum is
 * rounded to odd in binary64, and rounding that to 24 bits gives the
 * correctly rounded a*b + c (Boldo and Melquiond, "Emulation of FMA and
 * correctly rounded sums: proved algorithms using rounding to odd", IEEE
 * Trans. Computers 57(4), 2008: the odd rounding at p + 2 or more bits
 * followed by a nearest rounding at p bits equals one nearest rounding).
 * All binary64 values involved are normal, so the SSE flush modes leave
 * them alone.  (The operands are read as zeros explicitly; under DAZ the
 * conversion to binary64 would do the same.) */
static float f_daz(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0) u &= 0x80000000u;
    memcpy(&x, &u, 4);
    return x;
}

static double sum_round_to_odd(double p, double c) {
    double s = p + c;                            /* nearest */
    double bp = s - p;
    double err = (p - (s - bp)) + (c - bp);      /* p + c - s exactly (Knuth's TwoSum) */
    if (err != 0.0) {
        uint64_t bits;
        memcpy(&bits, &s, 8);
        if ((bits & 1u) == 0) s = nextafter(s, err > 0.0 ? INFINITY : -INFINITY);
    }
    return s;
}

static float f_fma(float a, float b, float c) {
    a = f_daz(a);
    b = f_daz(b);
    c = f_daz(c);
    const double s = sum_round_to_odd((double)a * (double)b, (double)c);
    if (s == 0.0) return (float)s;
    /* Round to 24 bits with an unbounded exponent: move tiny values into the
     * normal binary32 range by an exact power-of-two scaling first. */
    double r24;
    if (fabs(s) < 0x1p-64) r24 = (double)(float)(s * 0x1p+128) * 0x1p-128;
    else r24 = (double)(float)s;
    if (fabs(r24) < 0x1p-126) return s < 0.0 ? -0.0f : 0.0f;
    return (float)r24;
}

/* Elementwise fma under the contract, exported for the directed tests. */
int oracle_fma(const float* a, const float* b, const float* c, float* out, int64_t n) {
    if (n < 0) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    for (int64_t i = 0; i < n; ++i) out[i] = f_fma(a[i], b[i], c[i]);
    leave_contract(e);
    return ORACLE_OK;
}

/* GEMM under the fused convention: the same chains in the same order as
 * oracle_gemm, each step acc <- fma(a_ik, b_kj, acc), starting from +0. */
int oracle_gemm_fma(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                    const float* A, int64_t lda, const float* B, int64_t ldb,
                    float* C, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0) return ORACLE_EINVAL;
    if (M == 0 || N == 0) return ORACLE_OK;
    if (ldc < N) return ORACLE_EINVAL;
    if (K > 0) {
        if (lda < (trans_a ? M : K) || ldb < (trans_b ? K : N)) return ORACLE_EINVAL;
    }
    fpenv_t e = enter_contract();
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float a = trans_a ? A[k * lda + i] : A[i * lda + k];
                float b = trans_b ? B[j * ldb + k] : B[k * ldb + j];
                acc = f_fma(a, b, acc);
            }
            C[i * ldc + j] = acc;
        }
    }
    leave_contract(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* TreeFold (Appendix A.1, Algorithm 2) over whole replica vectors.
 *
 * Push(part): starting at level 0, while the stack's top entry has the same
 * level, pop it and set part = lower + part (the earlier, lower-replica block
 * is the left operand), then go one level up; finally push (level, part).
 * Result: take the partial of the lowest-level entry left on the stack, then
 * add every other remaining entry to it, in ascending level order.
 *
 * The average (Appendix A.3) multiplies by r = fl(1 / R), a binary32
 * reciprocal computed on the host, instead of dividing by R. */

typedef struct {
    int level;
    float* part;
} fold_entry_t;

typedef struct {
    fold_entry_t* stack;
    int depth;        /* entries in use */
    int capacity;
    int max_depth;    /* high-water mark of resident partials, incoming one included */
    int64_t n;
} treefold_t;

static void fold_push(treefold_t* f, float* part /* owned by the fold after the call */) {
    /* Resident partials at this moment: the stack plus the incoming one. */
    if (f->depth + 1 > f->max_depth) f->max_depth = f->depth + 1;
    int level = 0;
    while (f->depth > 0 && f->stack[f->depth - 1].level == level) {
        fold_entry_t lower = f->stack[--f->depth];
        for (int64_t i = 0; i < f->n; ++i) part[i] = f_add(lower.part[i], part[i]);
        free(lower.part);
        ++level;
    }
    f->stack[f->depth].level = level;
    f->stack[f->depth].part = part;
    ++f->depth;
}

/* Returns the running sum and releases the stack.  Entries sit on the stack
 * with strictly decreasing levels from bottom to top, so the lowest-level
 * entry is the top one and ascending level order walks down the stack. */
static float* fold_result(treefold_t* f) {
    float* acc = f->stack[f->depth - 1].part;
    for (int s = f->depth - 2; s >= 0; --s) {
        for (int64_t i = 0; i < f->n; ++i) acc[i] = f_add(acc[i], f->stack[s].part[i]);
        free(f->stack[s].part);
    }
    f->depth = 0;
    return acc;
}

/* out[i] = Fold(replicas[0][i], ..., replicas[R-1][i]), times fl(1/R) when
 * `average` is set.  With one replica the fold performs no operation, so
 * without the average the output is a copy of the input words.  max_resident (optional) receives the largest number of
 * partial vectors the fold held at once. */
int oracle_tree_reduce(const float* const* replicas, int32_t R, int64_t n, float* out,
                       int32_t average, int32_t* max_resident) {
    if (R < 1 || n < 0 || replicas == NULL) return ORACLE_EINVAL;
    for (int32_t r = 0; r < R; ++r) if (n > 0 && replicas[r] == NULL) return ORACLE_EINVAL;
    if (max_resident) *max_resident = 0;
    if (n == 0) return ORACLE_OK;
    fpenv_t e = enter_contract();
    treefold_t f;
    f.capacity = 40;
    f.stack = (fold_entry_t*)calloc((size_t)f.capacity, sizeof(fold_entry_t));
    f.depth = 0;
    f.max_depth = 0;
    f.n = n;
    if (!f.stack) { leave_contract(e); return ORACLE_ENOMEM; }
    for (int32_t r = 0; r < R; ++r) {
        float* part = (float*)malloc((size_t)n * sizeof(float));
        if (!part) { leave_contract(e); return ORACLE_ENOMEM; }
        for (int64_t i = 0; i < n; ++i) part[i] = replicas[r][i];
        fold_push(&f, part);
    }
    float* acc = fold_result(&f);
    if (average) {
        const float rR = f_div(1.0f, (float)R);
        for (int64_t i = 0; i < n; ++i) out[i] = f_mul(acc[i], rR);
    } else {
        for (int64_t i = 0; i < n; ++i) out[i] = acc[i];
    }
    if (max_resident) *max_resident = f.max_depth;
    free(acc);
    free(f.stack);
    leave_contract(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Audit replay of one step's gradient reduction (section 6, Algorithm 1, with
 * Appendix A.1-A.3).  N = dp_replicate * dp_shard virtual ranks in mesh order
 * (r = rep * dp_shard + shard); rank r has `accum` microbatch gradients,
 * grads[r * accum + k].  For every rank: g_r = 0, then for each microbatch
 * g_r = g_r + grad * fl(1/accum).  The shards of a replica are summed in
 * ascending shard order (inner = g_0, then inner = inner + g_s), the sum is
 * multiplied by fl(1/dp_shard) and pushed into the TreeFold; at the end the
 * fold's Result is multiplied by fl(1/dp_replicate).  Every "/" of the
 * algorithm is this multiply by a host-computed binary32 reciprocal
 * (Appendix A.3). */
int oracle_replay_reduce(const float* const* grads, int32_t dp_replicate, int32_t dp_shard, int32_t accum,
                         int64_t n, float* out) {
    if (dp_replicate < 1 || dp_shard < 1 || accum < 1 || n < 0 || grads == NULL) return ORACLE_EINVAL;
    const int64_t N = (int64_t)dp_replicate * dp_shard;
    for (int64_t b = 0; b < N * accum; ++b) if (n > 0 && grads[b] == NULL) return ORACLE_EINVAL;
    if (n == 0) return ORACLE_OK;
    fpenv_t e = enter_contract();
    const float r_accum = f_div(1.0f, (float)accum);
    const float r_shard = f_div(1.0f, (float)dp_shard);
    const float r_rep = f_div(1.0f, (float)dp_replicate);
    treefold_t f;
    f.capacity = 40;
    f.stack = (fold_entry_t*)calloc((size_t)f.capacity, sizeof(fold_entry_t));
    f.depth = 0;
    f.max_depth = 0;
    f.n = n;
    float* g = (float*)malloc((size_t)n * sizeof(float));
    float* inner = NULL;
    if (!f.stack || !g) { free(f.stack); free(g); leave_contract(e); return ORACLE_ENOMEM; }
    for (int64_t r = 0; r < N; ++r) {
        const int64_t shard = r % dp_shard;
        for (int64_t i = 0; i < n; ++i) g[i] = 0.0f;
        for (int32_t k = 0; k < accum; ++k) {
            const float* x = grads[r * accum + k];
            for (int64_t i = 0; i < n; ++i) g[i] = f_add(g[i], f_mul(x[i], r_accum));
        }
        if (shard == 0) {
            inner = (float*)malloc((size_t)n * sizeof(float));
            if (!inner) { free(g); leave_contract(e); return ORACLE_ENOMEM; }
            for (int64_t i = 0; i < n; ++i) inner[i] = g[i];
        } else {
            for (int64_t i = 0; i < n; ++i) inner[i] = f_add(inner[i], g[i]);
        }
        if (shard == dp_shard - 1) {
            for (int64_t i = 0; i < n; ++i) inner[i] = f_mul(inner[i], r_shard);
            fold_push(&f, inner); /* the fold owns `inner` from here */
            inner = NULL;
        }
    }
    float* acc = fold_result(&f);
    for (int64_t i = 0; i < n; ++i) out[i] = f_mul(acc[i], r_rep);
    free(acc);
    free(g);
    free(f.stack);
    leave_contract(e);
    return ORACLE_OK;
}

/* TreeFold as a streaming interface over caller-owned level slots (Appendix
 * A.1: at most floor(log2 R) + 1 partials resident).  slots[L] holds the
 * stack entry of level L, which exists exactly when bit L of `pushed` (the
 * number of partials pushed so far) is set.  Push combines the incoming
 * partial with the entries of levels 0, 1, ... while those bits are set
 * (lower block on the left) and stores the result in the first free level. */
int oracle_fold_push(float* const* slots, int32_t pushed, const float* part, int64_t n) {
    if (pushed < 0 || n < 0 || slots == NULL || (n > 0 && part == NULL)) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    int level = 0;
    float* carry = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!carry) { leave_contract(e); return ORACLE_ENOMEM; }
    for (int64_t i = 0; i < n; ++i) carry[i] = part[i];
    while ((pushed >> level) & 1) {
        for (int64_t i = 0; i < n; ++i) carry[i] = f_add(slots[level][i], carry[i]);
        ++level;
    }
    for (int64_t i = 0; i < n; ++i) slots[level][i] = carry[i];
    free(carry);
    leave_contract(e);
    return ORACLE_OK;
}

/* Result after `pushed` partials: start from the lowest occupied level and
 * add the others in ascending level order; multiply by fl(1/divisor) when
 * divisor > 0. */
int oracle_fold_result(float* const* slots, int32_t pushed, int64_t n, float* out, int32_t divisor) {
    if (pushed < 1 || n < 0 || slots == NULL || divisor < 0) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    int level = 0;
    while (((pushed >> level) & 1) == 0) ++level;
    for (int64_t i = 0; i < n; ++i) out[i] = slots[level][i];
    for (int L = level + 1; L < 31; ++L) {
        if ((pushed >> L) & 1) {
            for (int64_t i = 0; i < n; ++i) out[i] = f_add(out[i], slots[L][i]);
        }
    }
    if (divisor > 0) {
        const float r = f_div(1.0f, (float)divisor);
        for (int64_t i = 0; i < n; ++i) out[i] = f_mul(out[i], r);
    }
    leave_contract(e);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* AdamW (Loshchilov and Hutter), as the fused FP32 optimizer step of the
 * OPEN-1B recipe, section 3.2.  State is one flat array [w | m | v] of 3n
 * binary32 words (checkpoint page, "file format"); grad has n words.
 *
 * Host scalars, each one binary32 contract operation:
 *   c1 = 1 - beta1, c2 = 1 - beta2;
 *   p1 = beta1^t as t-1 serial multiplies starting from beta1, p2 likewise;
 *   bc1 = 1 - p1, bc2 = 1 - p2; r1 = 1 / bc1, r2 = 1 / bc2.
 * Per element, in this order:
 *   m' = beta1*m + c1*g
 *   v' = beta2*v + c2*(g*g)
 *   mh = m' * r1,  vh = v' * r2
 *   u  = mh / (sqrt(vh) + eps)
 *   w' = w - lr * (u + wd * w)
 */
typedef struct { float c1, c2, r1, r2; } adamw_scalars_t;

static adamw_scalars_t adamw_host_scalars(float beta1, float beta2, int64_t step) {
    adamw_scalars_t s;
    s.c1 = f_sub(1.0f, beta1);
    s.c2 = f_sub(1.0f, beta2);
    float p1 = beta1, p2 = beta2;
    for (int64_t t = 1; t < step; ++t) {
        p1 = f_mul(p1, beta1);
        p2 = f_mul(p2, beta2);
    }
    float bc1 = f_sub(1.0f, p1), bc2 = f_sub(1.0f, p2);
    s.r1 = f_div(1.0f, bc1);
    s.r2 = f_div(1.0f, bc2);
    return s;
}

/* One element of the update: the 16 operations in the order above. */
static void adamw_element(float w, float m, float v, float g, adamw_scalars_t s, float lr, float beta1,
                          float beta2, float eps, float weight_decay, float* w_out, float* m_out, float* v_out) {
    const float m1 = f_mul(beta1, m);
    const float m2 = f_mul(s.c1, g);
    const float mn = f_add(m1, m2);
    const float q = f_mul(g, g);
    const float v1 = f_mul(beta2, v);
    const float v2 = f_mul(s.c2, q);
    const float vn = f_add(v1, v2);
    const float mh = f_mul(mn, s.r1);
    const float vh = f_mul(vn, s.r2);
    const float sq = f_sqrt(vh);
    const float d = f_add(sq, eps);
    const float u = f_div(mh, d);
    const float y = f_mul(weight_decay, w);
    const float z = f_add(u, y);
    const float t = f_mul(lr, z);
    const float wn = f_sub(w, t);
    *w_out = wn;
    *m_out = mn;
    *v_out = vn;
}

int oracle_adamw_scalars(float beta1, float beta2, int64_t step, float out4[4]) {
    if (step < 1) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    adamw_scalars_t s = adamw_host_scalars(beta1, beta2, step);
    out4[0] = s.c1; out4[1] = s.c2; out4[2] = s.r1; out4[3] = s.r2;
    leave_contract(e);
    return ORACLE_OK;
}

int oracle_adamw(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2,
                 float eps, float weight_decay, int64_t step) {
    if (n < 0 || step < 1) return ORACLE_EINVAL;
    if (n == 0) return ORACLE_OK;
    fpenv_t e = enter_contract();
    const adamw_scalars_t s = adamw_host_scalars(beta1, beta2, step);
    float* W = state;
    float* Mo = state + n;
    float* V = state + 2 * n;
    for (int64_t i = 0; i < n; ++i) {
        const float g = grad[i], w = W[i], m = Mo[i], v = V[i];
        float wn, mn, vn;
        adamw_element(w, m, v, g, s, lr, beta1, beta2, eps, weight_decay, &wn, &mn, &vn);
        W[i] = wn;
        Mo[i] = mn;
        V[i] = vn;
    }
    leave_contract(e);
    return ORACLE_OK;
}
/* ------------------------------------------------------------------------ */
/* BF16 parameters (section 3.1: parameters held in BF16; section 3.2
 * "Optimizer-state precision": the fused step widens the BF16 parameter and
 * gradient to FP32, updates in FP32 with FP32 moments, and rounds the
 * parameter back to BF16 once).  With the global-norm clip (section 3.2,
 * "Optimizer": gradients clipped to a global l2 norm of 1.0) and the spike
 * protocol (section 3.4.2: five optimizer steps are skipped when the
 * pre-clip gradient norm exceeds 5). */

/* bf16 -> binary32: the 16 bits are the high half of the binary32 word. */
static float bf16_widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static double f32_bits_to_double(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even: of the two bf16 values
 * around x (x truncated toward zero, and the next one away from zero) take
 * the nearer, by exact binary64 distances; on a tie take the one whose last
 * kept bit is 0 (past the largest bf16 this gives infinity, as IEEE does).  x is a normal binary32 value or a zero here (every result
 * of the update is), so the rounded value is never below 2^-126 unless it is
 * a zero, and the flush rule has nothing to do. */
static uint16_t bf16_round(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    const uint32_t lo = u & 0xFFFF0000u;
    const uint32_t hi = lo + 0x10000u;
    const double ax = fabs((double)x);
    const double dlo = ax - fabs(f32_bits_to_double(lo));
    /* Above the largest bf16 the next value is infinity; the rounding
     * compares with 2^128, where the unbounded-exponent grid continues
     * (IEEE 754 overflow: round as if the exponent were unbounded). */
    const double vhi = ((hi >> 23) & 0xFFu) == 0xFFu ? 0x1p+128 : fabs(f32_bits_to_double(hi));
    const double dhi = vhi - ax;
    uint32_t r;
    if (dlo < dhi) r = lo;
    else if (dhi < dlo) r = hi;
    else r = ((lo >> 16) & 1u) == 0 ? lo : hi;
    return (uint16_t)(r >> 16);
}

static float load_grad(const void* g, int dtype, int64_t i) {
    return dtype == 1 ? bf16_widen(((const uint16_t*)g)[i]) : ((const float*)g)[i];
}

/* Global l2 norm of the gradient, as the pre-clip norm: q_i = g_i * g_i
 * (binary32, widened first for bf16), S = TreeFold over q_0 .. q_{n-1} in
 * index order (Appendix A.1's fold, applied to scalars: blocks combined as in
 * binary counting, lower block on the left, Result from the lowest level
 * upward), norm = sqrt(S) correctly rounded.  S = 0 for n = 0. */
static float grad_norm_of(const void* g, int dtype, int64_t n, float* sumsq) {
    float val[64];
    int lvl[64];
    int depth = 0;
    for (int64_t i = 0; i < n; ++i) {
        const float x = load_grad(g, dtype, i);
        float part = f_mul(x, x);
        int level = 0;
        while (depth > 0 && lvl[depth - 1] == level) {
            part = f_add(val[depth - 1], part);
            --depth;
            ++level;
        }
        val[depth] = part;
        lvl[depth] = level;
        ++depth;
    }
    float acc = 0.0f;
    if (depth > 0) {
        acc = val[depth - 1];
        for (int d = depth - 2; d >= 0; --d) acc = f_add(acc, val[d]);
    }
    if (sumsq) *sumsq = acc;
    return f_sqrt(acc);
}

/* out2[0] = the norm, out2[1] = S, the fold of the squares. */
int oracle_grad_norm(const void* g, int32_t dtype, int64_t n, float* out2) {
    if (n < 0 || (dtype != 0 && dtype != 1) || (n > 0 && g == NULL)) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    out2[0] = grad_norm_of(g, dtype, n, &out2[1]);
    leave_contract(e);
    return ORACLE_OK;
}

/* The optimizer-step record kept between steps (mirrors the library's
 * layout field for field; the oracle has its own definition). */
typedef struct {
    int64_t step;      /* updates applied so far */
    int32_t skip_left; /* steps still to skip */
    int32_t applied;   /* 1 if the last step applied its update */
    float beta1_pow;   /* beta1^step (any value while step == 0) */
    float beta2_pow;
    float grad_norm;   /* the last step's pre-clip norm */
    float clip_coef;   /* the coefficient applied to the gradient (1 if none) */
} oracle_step_state_t;

/* One optimizer step on bf16 parameters w[n], FP32 moments m[n], v[n] and a
 * gradient g[n] (dtype 0 binary32, 1 bf16), following the recipe:
 *   norm = the pre-clip global norm above
 *   spike rule (spike_threshold > 0): norm > spike_threshold starts a
 *     window of skip_steps skipped steps, this one included (a spike inside
 *     a window starts it again);
 *   a skipped step changes neither w, m, v nor the step count;
 *   clip (max_norm > 0): coef = max_norm / (norm + 1e-6); if coef < 1 every
 *     gradient element is multiplied by it, one binary32 product each;
 *   an applied step is step t = step + 1, with beta^t carried as one more
 *     serial multiply (beta itself at t = 1) and the host scalars of the
 *     FP32 update, which then runs on (widen(w), m, v, g) and rounds w' to
 *     bf16 once. */
int oracle_adamw_bf16_step(uint16_t* w, float* m, float* v, const void* g, int32_t dtype, int64_t n, float lr,
                           float beta1, float beta2, float eps, float weight_decay, float max_norm,
                           float spike_threshold, int32_t skip_steps, oracle_step_state_t* st) {
    if (n < 0 || (dtype != 0 && dtype != 1) || skip_steps < 0 || st == NULL) return ORACLE_EINVAL;
    if (n > 0 && (w == NULL || m == NULL || v == NULL || g == NULL)) return ORACLE_EINVAL;
    fpenv_t e = enter_contract();
    const float norm = grad_norm_of(g, dtype, n, NULL);
    st->grad_norm = norm;
    if (spike_threshold > 0.0f && norm > spike_threshold) st->skip_left = skip_steps;
    int apply = 1;
    if (st->skip_left > 0) {
        apply = 0;
        st->skip_left -= 1;
    }
    float coef = 1.0f;
    if (max_norm > 0.0f) {
        const float c = f_div(max_norm, f_add(norm, 1e-6f));
        if (c < 1.0f) coef = c;
    }
    st->clip_coef = coef;
    st->applied = apply;
    if (apply) {
        const int64_t t = st->step + 1;
        const float p1 = t == 1 ? beta1 : f_mul(st->beta1_pow, beta1);
        const float p2 = t == 1 ? beta2 : f_mul(st->beta2_pow, beta2);
        adamw_scalars_t s;
        s.c1 = f_sub(1.0f, beta1);
        s.c2 = f_sub(1.0f, beta2);
        s.r1 = f_div(1.0f, f_sub(1.0f, p1));
        s.r2 = f_div(1.0f, f_sub(1.0f, p2));
        for (int64_t i = 0; i < n; ++i) {
            float gi = load_grad(g, dtype, i);
            if (coef < 1.0f) gi = f_mul(gi, coef);
            float wn, mn, vn;
            adamw_element(bf16_widen(w[i]), m[i], v[i], gi, s, lr, beta1, beta2, eps, weight_decay, &wn, &mn, &vn);
            w[i] = bf16_round(wn);
            m[i] = mn;
            v[i] = vn;
        }
        st->step = t;
        st->beta1_pow = p1;
        st->beta2_pow = p2;
    }
    leave_contract(e);
    return ORACLE_OK;
}

/* Exported for the pins: bf16 rounding and widening of n values. */
int oracle_bf16_round(const float* x, uint16_t* out, int64_t n) {
    if (n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(x[i]);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* BLAKE2b, RFC 7693, with the tree-hashing parameter block of the BLAKE2
 * paper (Aumasson, Neves, Wilcox-O'Hearn, Winnerlein, 2013, section 2.10). */

static const uint64_t B2B_IV[8] = {
    0x6A09E667F3BCC908ULL, 0xBB67AE8584CAA73BULL, 0x3C6EF372FE94F82BULL, 0xA54FF53A5F1D36F1ULL,
    0x510E527FADE682D1ULL, 0x9B05688C2B3E6C1FULL, 0x1F83D9ABFB41BD6BULL, 0x5BE0CD19137E2179ULL};

static const uint8_t B2B_SIGMA[12][16] = {
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15},
    {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3},
    {11, 8, 12, 0, 5, 2, 15, 13, 10, 14, 3, 6, 7, 1, 9, 4},
    {7, 9, 3, 1, 13, 12, 11, 14, 2, 6, 5, 10, 4, 0, 15, 8},
    {9, 0, 5, 7, 2, 4, 10, 15, 14, 1, 11, 12, 6, 8, 3, 13},
    {2, 12, 6, 10, 0, 11, 8, 3, 4, 13, 7, 5, 15, 14, 1, 9},
    {12, 5, 1, 15, 14, 13, 4, 10, 0, 7, 6, 3, 9, 2, 8, 11},
    {13, 11, 7, 14, 12, 1, 3, 9, 5, 0, 15, 4, 8, 6, 2, 10},
    {6, 15, 14, 9, 11, 3, 0, 8, 12, 2, 13, 7, 1, 4, 10, 5},
    {10, 2, 8, 4, 7, 6, 1, 5, 15, 11, 9, 14, 3, 12, 13, 0},
    {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15},
    {14, 10, 4, 8, 9, 15, 13, 6, 1, 12, 0, 2, 11, 7, 5, 3}};

static uint64_t rotr64(uint64_t x, int r) { return (x >> r) | (x << (64 - r)); }

static uint64_t load_le64(const uint8_t* p) {
    uint64_t x = 0;
    for (int i = 7; i >= 0; --i) x = (x << 8) | p[i];
    return x;
}

static void store_le64(uint8_t* p, uint64_t x) {
    for (int i = 0; i < 8; ++i) { p[i] = (uint8_t)(x & 0xFF); x >>= 8; }
}

typedef struct {
    uint64_t h[8];
    uint64_t t0, t1;  /* byte counter, low and high words */
    uint8_t buf[128];
    size_t buflen;
    int last_node;
    int outlen;
} b2b_t;

static void b2b_compress(b2b_t* s, const uint8_t block[128], int last_block) {
    uint64_t m[16], v[16];
    for (int i = 0; i < 16; ++i) m[i] = load_le64(block + 8 * i);
    for (int i = 0; i < 8; ++i) { v[i] = s->h[i]; v[i + 8] = B2B_IV[i]; }
    v[12] ^= s->t0;
    v[13] ^= s->t1;
    if (last_block) {
        v[14] = ~v[14];
        if (s->last_node) v[15] = ~v[15];
    }
#define G(a, b, c, d, x, y)                 \
    do {                                    \
        v[a] = v[a] + v[b] + (x);           \
        v[d] = rotr64(v[d] ^ v[a], 32);     \
        v[c] = v[c] + v[d];                 \
        v[b] = rotr64(v[b] ^ v[c], 24);     \
        v[a] = v[a] + v[b] + (y);           \
        v[d] = rotr64(v[d] ^ v[a], 16);     \
        v[c] = v[c] + v[d];                 \
        v[b] = rotr64(v[b] ^ v[c], 63);     \
    } while (0)
    for (int r = 0; r < 12; ++r) {
        const uint8_t* sg = B2B_SIGMA[r];
        G(0, 4, 8, 12, m[sg[0]], m[sg[1]]);
        G(1, 5, 9, 13, m[sg[2]], m[sg[3]]);
        G(2, 6, 10, 14, m[sg[4]], m[sg[5]]);
        G(3, 7, 11, 15, m[sg[6]], m[sg[7]]);
        G(0, 5, 10, 15, m[sg[8]], m[sg[9]]);
        G(1, 6, 11, 12, m[sg[10]], m[sg[11]]);
        G(2, 7, 8, 13, m[sg[12]], m[sg[13]]);
        G(3, 4, 9, 14, m[sg[14]], m[sg[15]]);
    }
#undef G
    for (int i = 0; i < 8; ++i) s->h[i] ^= v[i] ^ v[i + 8];
}

/* Parameter block: byte 0 digest length, 1 key length, 2 fanout, 3 depth,
 * 4..7 leaf length, 8..15 node offset, 16 node depth, 17 inner length,
 * 18..31 reserved, 32..47 salt, 48..63 personalisation (all little-endian). */
static void b2b_init_param(b2b_t* s, int outlen, int fanout, int depth, uint32_t leaf_length,
                           uint64_t node_offset, int node_depth, int inner_length,
                           const uint8_t personal[16], int last_node) {
    uint8_t p[64];
    memset(p, 0, sizeof p);
    p[0] = (uint8_t)outlen;
    p[1] = 0;
    p[2] = (uint8_t)fanout;
    p[3] = (uint8_t)depth;
    for (int i = 0; i < 4; ++i) p[4 + i] = (uint8_t)(leaf_length >> (8 * i));
    for (int i = 0; i < 8; ++i) p[8 + i] = (uint8_t)(node_offset >> (8 * i));
    p[16] = (uint8_t)node_depth;
    p[17] = (uint8_t)inner_length;
    if (personal) memcpy(p + 48, personal, 16);
    for (int i = 0; i < 8; ++i) s->h[i] = B2B_IV[i] ^ load_le64(p + 8 * i);
    s->t0 = s->t1 = 0;
    s->buflen = 0;
    s->last_node = last_node;
    s->outlen = outlen;
}

static void b2b_update(b2b_t* s, const uint8_t* in, size_t len) {
    while (len > 0) {
        if (s->buflen == 128) {
            /* A full block is only compressed once more input follows, so the
             * final block is always compressed with the last-block flag. */
            s->t0 += 128;
            if (s->t0 < 128) s->t1++;
            b2b_compress(s, s->buf, 0);
            s->buflen = 0;
        }
        size_t take = 128 - s->buflen;
        if (take > len) take = len;
        memcpy(s->buf + s->buflen, in, take);
        s->buflen += take;
        in += take;
        len -= take;
    }
}

static void b2b_final(b2b_t* s, uint8_t* out) {
    s->t0 += s->buflen;
    if (s->t0 < s->buflen) s->t1++;
    memset(s->buf + s->buflen, 0, 128 - s->buflen);
    b2b_compress(s, s->buf, 1);
    uint8_t full[64];
    for (int i = 0; i < 8; ++i) store_le64(full + 8 * i, s->h[i]);
    memcpy(out, full, (size_t)s->outlen);
}

/* Plain (sequential-mode) BLAKE2b with an optional personalisation, for the
 * RFC 7693 known-answer pin. */
int oracle_blake2b(const uint8_t* in, int64_t len, int outlen, const uint8_t* personal16, uint8_t* out) {
    if (len < 0 || outlen < 1 || outlen > 64) return ORACLE_EINVAL;
    b2b_t s;
    b2b_init_param(&s, outlen, 1, 1, 0, 0, 0, 0, personal16, 0);
    b2b_update(&s, in, (size_t)len);
    b2b_final(&s, out);
    return ORACLE_OK;
}

/* State hash: BLAKE2b tree mode over the little-endian bytes of the words.
 *   digest 32 bytes; fanout 16; depth 255; leaf length 4096; inner 32;
 *   personalisation "repro_state_v1" padded with zero bytes to 16.
 * Level 0: the bytes are cut into leaves of 4096 bytes (the last one may be
 * shorter; an empty input is one empty leaf).  Leaf i is hashed with node
 * offset i, node depth 0, and the last-node flag on the last leaf only.
 * Level d >= 1: node j hashes the concatenated 32-byte digests of children
 * 16j .. 16j+15 of level d-1, node offset j, node depth d, last-node flag
 * on the last node of the level.  Levels are added until one node is left;
 * there is always at least one level above the leaves.  That node is the
 * root and its digest is the state hash. */
#define SH_LEAF 4096
#define SH_FANOUT 16
#define SH_DEPTH 255
#define SH_INNER 32
static const uint8_t SH_PERSONAL[16] = {'r', 'e', 'p', 'r', 'o', '_', 's', 't', 'a', 't', 'e', '_', 'v', '1', 0, 0};

static void sh_node(const uint8_t* in, size_t len, uint64_t offset, int depth, int last, uint8_t out[32]) {
    b2b_t s;
    b2b_init_param(&s, SH_INNER, SH_FANOUT, SH_DEPTH, SH_LEAF, offset, depth, SH_INNER, SH_PERSONAL, last);
    b2b_update(&s, in, len);
    b2b_final(&s, out);
}

/* Leaf digests only (level 0), for checking sampled leaves of large inputs. */
int oracle_state_hash_leaves(const float* words, int64_t n_words, int64_t leaf0, int64_t count,
                             uint8_t* out32) {
    if (n_words < 0 || leaf0 < 0 || count < 0) return ORACLE_EINVAL;
    const uint64_t nbytes = (uint64_t)n_words * 4u;
    const int64_t leaves = nbytes == 0 ? 1 : (int64_t)((nbytes + SH_LEAF - 1) / SH_LEAF);
    if (leaf0 + count > leaves) return ORACLE_EINVAL;
    const uint8_t* bytes = (const uint8_t*)words;  /* x86 is little-endian */
    for (int64_t i = leaf0; i < leaf0 + count; ++i) {
        uint64_t b = (uint64_t)i * SH_LEAF;
        uint64_t len = nbytes - b < SH_LEAF ? nbytes - b : SH_LEAF;
        if (nbytes == 0) len = 0;
        sh_node(bytes + b, (size_t)len, (uint64_t)i, 0, i == leaves - 1, out32 + 32 * (i - leaf0));
    }
    return ORACLE_OK;
}

/* One leaf on its own: `n_words` words (at most 1024) hashed as leaf number
 * `leaf` of a tree, with the last-node flag when `last` is set. */
int oracle_state_hash_one_leaf(const float* words, int64_t n_words, int64_t leaf, int last, uint8_t* out32) {
    if (n_words < 0 || n_words * 4 > SH_LEAF || leaf < 0) return ORACLE_EINVAL;
    sh_node((const uint8_t*)words, (size_t)n_words * 4, (uint64_t)leaf, 0, last != 0, out32);
    return ORACLE_OK;
}

int oracle_state_hash(const float* words, int64_t n_words, uint8_t digest[32]) {
    if (n_words < 0) return ORACLE_EINVAL;
    const uint64_t nbytes = (uint64_t)n_words * 4u;
    int64_t count = nbytes == 0 ? 1 : (int64_t)((nbytes + SH_LEAF - 1) / SH_LEAF);
    uint8_t* level = (uint8_t*)malloc((size_t)count * 32);
    if (!level) return ORACLE_ENOMEM;
    int rc = oracle_state_hash_leaves(words, n_words, 0, count, level);
    if (rc != ORACLE_OK) { free(level); return rc; }
    int depth = 1;
    do {
        int64_t parents = (count + SH_FANOUT - 1) / SH_FANOUT;
        uint8_t* up = (uint8_t*)malloc((size_t)parents * 32);
        if (!up) { free(level); return ORACLE_ENOMEM; }
        for (int64_t j = 0; j < parents; ++j) {
            int64_t c0 = j * SH_FANOUT;
            int64_t nc = count - c0 < SH_FANOUT ? count - c0 : SH_FANOUT;
            sh_node(level + 32 * c0, (size_t)nc * 32, (uint64_t)j, depth, j == parents - 1, up + 32 * j);
        }
        free(level);
        level = up;
        count = parents;
        ++depth;
    } while (count > 1);
    memcpy(digest, level, 32);
    free(level);
    return ORACLE_OK;
}

const char* oracle_spec_version(void) { return "repro-spec-1"; }
