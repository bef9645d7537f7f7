/* Calls every entry point of the CPU oracle on small, edge-case inputs, so
 * that a build with AddressSanitizer and UndefinedBehaviorSanitizer can check
 * its memory accesses and integer arithmetic.  Test infrastructure: built and
 * run by tests/test_oracle_sanitized.py on the host only.  Exit status 0 when
 * every call returned its expected status. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fp32_ops(int op, const float* a, const float* b, float* out, int64_t n);
int oracle_gemm(int ta, int tb, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                int64_t ldb, float* C, int64_t ldc);
int oracle_gemm_fma(int ta, int tb, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
                    int64_t ldb, float* C, int64_t ldc);
int oracle_fma(const float* a, const float* b, const float* c, float* out, int64_t n);
int oracle_tree_reduce(const float* const* replicas, int32_t R, int64_t n, float* out, int32_t average,
                       int32_t* max_resident);
int oracle_replay_reduce(const float* const* grads, int32_t dp_replicate, int32_t dp_shard, int32_t accum,
                         int64_t n, float* out);
int oracle_fold_push(float* const* slots, int32_t pushed, const float* part, int64_t n);
int oracle_fold_result(float* const* slots, int32_t pushed, int64_t n, float* out, int32_t divisor);
int oracle_adamw_scalars(float beta1, float beta2, int64_t step, float out4[4]);
int oracle_adamw(float* state, const float* grad, int64_t n, float lr, float beta1, float beta2, float eps,
                 float weight_decay, int64_t step);
int oracle_grad_norm(const void* g, int32_t dtype, int64_t n, float* out2);
int oracle_adamw_bf16_step(uint16_t* w, float* m, float* v, const void* g, int32_t dtype, int64_t n, float lr,
                           float beta1, float beta2, float eps, float weight_decay, float max_norm,
                           float spike_threshold, int32_t skip_steps, void* st);
int oracle_bf16_round(const float* x, uint16_t* out, int64_t n);
int oracle_blake2b(const uint8_t* in, int64_t len, int outlen, const uint8_t* personal16, uint8_t* out);
int oracle_state_hash_leaves(const float* words, int64_t n_words, int64_t leaf0, int64_t count, uint8_t* out32);
int oracle_state_hash_one_leaf(const float* words, int64_t n_words, int64_t leaf, int last, uint8_t* out32);
int oracle_state_hash(const float* words, int64_t n_words, uint8_t digest[32]);

static int failures = 0;
#define EXPECT(call, status)                                                      \
    do {                                                                          \
        int rc_ = (call);                                                         \
        if (rc_ != (status)) {                                                    \
            fprintf(stderr, "%s:%d: %s returned %d\n", __FILE__, __LINE__, #call, rc_); \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

/* Exactly-sized heap buffers, so that ASan sees any access past the end. */
static float* fbuf(int64_t n, unsigned seed) {
    float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) {
        seed = seed * 1664525u + 1013904223u;
        p[i] = (float)((int)(seed >> 8) % 2001 - 1000) * 0.001f;
    }
    return p;
}

int main(void) {
    /* fp32 contract operations */
    float* a = fbuf(17, 1);
    float* b = fbuf(17, 2);
    float* c = fbuf(17, 3);
    float* o = fbuf(17, 4);
    for (int op = 0; op <= 4; ++op) EXPECT(oracle_fp32_ops(op, a, b, o, 17), 0);
    EXPECT(oracle_fma(a, b, c, o, 17), 0);
    /* GEMM, both conventions, all transposes, ragged and empty shapes */
    const int64_t M = 3, N = 5, K = 7;
    for (int ta = 0; ta <= 1; ++ta)
        for (int tb = 0; tb <= 1; ++tb) {
            float* A = fbuf(M * K, 5);
            float* B = fbuf(K * N, 6);
            float* C = fbuf(M * N, 7);
            EXPECT(oracle_gemm(ta, tb, M, N, K, A, ta ? M : K, B, tb ? K : N, C, N), 0);
            EXPECT(oracle_gemm_fma(ta, tb, M, N, K, A, ta ? M : K, B, tb ? K : N, C, N), 0);
            EXPECT(oracle_gemm(ta, tb, M, N, 0, A, 1, B, 1, C, N), 0);
            free(A); free(B); free(C);
        }
    /* TreeFold over R replicas, R = 1 .. 9, and the replay */
    for (int R = 1; R <= 9; ++R) {
        float* reps[9];
        for (int r = 0; r < R; ++r) reps[r] = fbuf(13, 10 + r);
        float* out = fbuf(13, 30);
        int32_t resident = 0;
        EXPECT(oracle_tree_reduce((const float* const*)reps, R, 13, out, R % 2, &resident), 0);
        for (int r = 0; r < R; ++r) free(reps[r]);
        free(out);
    }
    {
        float* g[12];
        for (int i = 0; i < 12; ++i) g[i] = fbuf(11, 40 + i);
        float* out = fbuf(11, 60);
        EXPECT(oracle_replay_reduce((const float* const*)g, 2, 3, 2, 11, out), 0);
        for (int i = 0; i < 12; ++i) free(g[i]);
        free(out);
    }
    {
        float* slots[3];
        for (int L = 0; L < 3; ++L) slots[L] = fbuf(9, 70 + L);
        for (int i = 0; i < 5; ++i) {
            float* part = fbuf(9, 80 + i);
            EXPECT(oracle_fold_push(slots, i, part, 9), 0);
            free(part);
        }
        float* out = fbuf(9, 90);
        EXPECT(oracle_fold_result(slots, 5, 9, out, 5), 0);
        for (int L = 0; L < 3; ++L) free(slots[L]);
        free(out);
    }
    /* AdamW, FP32 and BF16 forms, and the norm */
    {
        float s4[4];
        EXPECT(oracle_adamw_scalars(0.9f, 0.999f, 1000, s4), 0);
        float* st = fbuf(27, 100);
        float* g = fbuf(9, 101);
        EXPECT(oracle_adamw(st, g, 9, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, 3), 0);
        EXPECT(oracle_adamw(st, g, 9, 1e-3f, 0.9f, 0.999f, 1e-8f, 0.1f, 0), -1);
        free(st); free(g);
        float norm2[2];
        float* gf = fbuf(4097, 102);
        EXPECT(oracle_grad_norm(gf, 0, 4097, norm2), 0);
        EXPECT(oracle_grad_norm(gf, 0, 0, norm2), 0);
        uint16_t* gh = (uint16_t*)malloc(4097 * sizeof(uint16_t));
        EXPECT(oracle_bf16_round(gf, gh, 4097), 0);
        EXPECT(oracle_grad_norm(gh, 1, 4097, norm2), 0);
        uint16_t* w = (uint16_t*)malloc(33 * sizeof(uint16_t));
        EXPECT(oracle_bf16_round(gf, w, 33), 0);
        float* m = fbuf(33, 103);
        float* v = fbuf(33, 104);
        for (int i = 0; i < 33; ++i) v[i] = v[i] * v[i];
        uint64_t state[4] = {0, 0, 0, 0}; /* 32 bytes, zero = fresh */
        for (int step = 0; step < 8; ++step)
            EXPECT(oracle_adamw_bf16_step(w, m, v, step == 2 ? (const void*)gf : (const void*)gh, step == 2 ? 0 : 1,
                                          33, 1e-3f, 0.9f, 0.95f, 1e-8f, 0.1f, 1.0f, 0.05f, 5, state), 0);
        free(gf); free(gh); free(w); free(m); free(v);
    }
    /* BLAKE2b and the state hash: empty, partial leaf, exact leaves, several levels */
    {
        uint8_t out[64];
        uint8_t* data = (uint8_t*)malloc(129);
        memset(data, 0x5a, 129);
        const uint8_t person[16] = {0};
        EXPECT(oracle_blake2b(data, 0, 64, person, out), 0);
        EXPECT(oracle_blake2b(data, 3, 32, person, out), 0);
        EXPECT(oracle_blake2b(data, 129, 64, person, out), 0);
        free(data);
        const int64_t sizes[] = {0, 1, 1023, 1024, 1025, 17 * 1024 + 5, 300 * 1024};
        for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) {
            float* words = fbuf(sizes[i], 200 + (unsigned)i);
            uint8_t digest[32];
            EXPECT(oracle_state_hash(words, sizes[i], digest), 0);
            const int64_t leaves = sizes[i] == 0 ? 1 : (sizes[i] + 1023) / 1024;
            uint8_t* d = (uint8_t*)malloc((size_t)leaves * 32);
            EXPECT(oracle_state_hash_leaves(words, sizes[i], 0, leaves, d), 0);
            free(d);
            const int64_t tail = sizes[i] - (leaves - 1) * 1024;
            EXPECT(oracle_state_hash_one_leaf(words + (leaves - 1) * 1024, tail, leaves - 1, 1, digest), 0);
            free(words);
        }
    }
    free(a); free(b); free(c); free(o);
    if (failures) fprintf(stderr, "%d failures\n", failures);
    return failures ? 1 : 0;
}
