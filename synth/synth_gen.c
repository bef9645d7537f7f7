/*
 * Seeded synthetic inputs for the reproducible-ops workloads.
 *
 * This module holds no arithmetic of the reproducible operations themselves:
 * it only turns (seed, tensor id, element index) into fp32 input values.  Both
 * the CPU oracle checks and the GPU path consume the same host buffers made
 * here.
 *
 * Generator: Philox4x64-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).  It is
 * the same function as numpy.random.Philox, which the tests use to check it.
 * A value is a pure function of (key, counter), so the output does not depend
 * on how the index range is split over threads.  The OPEN-1B paper (section
 * 2.1, "Random number generation"; Table 1) asks for exactly this kind of
 * position-indexed stream.
 *
 * Layout of one stream: key = (seed, tensor_id), counter = (block, sub, 0, 0)
 * where `sub` selects an independent sub-stream of the same tensor (mask,
 * replacement draw, Student-t chi-square parts).  Block b yields four 64-bit
 * words; element e of a stream uses word e % 4 of block e / 4.
 *
 * Uniform:  u = ((x >> 11) + 0.5) * 2^-53, in (0, 1), never 0 or 1.
 * Normal:   Box-Muller in binary64 on the word pairs (0,1) and (2,3) of a
 *           block: r = sqrt(-2 ln u_a), z_a = r cos(2 pi u_b),
 *           z_b = r sin(2 pi u_b).  Element 4b+0 gets the cosine of pair
 *           (0,1), 4b+1 its sine, 4b+2 and 4b+3 likewise from pair (2,3).
 * Every value is formed in binary64 and rounded to binary32 once.
 *
 * Build: gcc -O2 -fPIC -shared -pthread (see synth/build.py).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PHILOX_M0 0xD2E7470EE14C6C93ULL
#define PHILOX_M1 0xCA5A826395121157ULL
#define PHILOX_W0 0x9E3779B97F4A7C15ULL
#define PHILOX_W1 0xBB67AE8584CAA73BULL

static inline uint64_t mulhilo64(uint64_t a, uint64_t b, uint64_t* hi) {
    unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
    *hi = (uint64_t)(p >> 64);
    return (uint64_t)p;
}

/* Philox4x64 with 10 rounds; the key is bumped by the Weyl constants
 * between rounds. */
void synth_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
        uint64_t hi0, hi1;
        uint64_t lo0 = mulhilo64(PHILOX_M0, c0, &hi0);
        uint64_t lo1 = mulhilo64(PHILOX_M1, c2, &hi1);
        uint64_t n0 = hi1 ^ c1 ^ k0;
        uint64_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline double u01(uint64_t x) {
    return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Four standard normals from one counter block of stream (seed, tid, sub). */
static void normal4(uint64_t seed, uint64_t tid, uint64_t sub, uint64_t block, double z[4]) {
    const uint64_t key[2] = {seed, tid};
    const uint64_t ctr[4] = {block, sub, 0, 0};
    uint64_t w[4];
    synth_philox4x64_10(ctr, key, w);
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double ua = u01(w[2 * p]), ub = u01(w[2 * p + 1]);
        double r = sqrt(-2.0 * log(ua));
        z[2 * p] = r * cos(two_pi * ub);
        z[2 * p + 1] = r * sin(two_pi * ub);
    }
}

static void uniform4(uint64_t seed, uint64_t tid, uint64_t sub, uint64_t block, double u[4]) {
    const uint64_t key[2] = {seed, tid};
    const uint64_t ctr[4] = {block, sub, 0, 0};
    uint64_t w[4];
    synth_philox4x64_10(ctr, key, w);
    for (int i = 0; i < 4; ++i) u[i] = u01(w[i]);
}

/* Sub-stream numbers inside one tensor id. */
enum { SUB_MAIN = 0, SUB_MASK = 1, SUB_REPL = 2, SUB_CHI1 = 3, SUB_CHI2 = 4, SUB_CHI3 = 5 };

/* Distribution kinds.
 *  0 NORMAL          std * z
 *  1 HALF_NORMAL     |std * z|
 *  2 OUTLIER_SCALED  std * z, times p2 where a Bernoulli(p1) mask is set
 *  3 OUTLIER_REPLACE std * z, replaced by p2 * z' where a Bernoulli(p1) mask is set
 *  4 STUDENT_T3      std * z / sqrt((z1^2 + z2^2 + z3^2) / 3)
 *  5 UNIFORM         std * (2u - 1)
 */
enum { K_NORMAL = 0, K_HALF_NORMAL = 1, K_OUTLIER_SCALED = 2, K_OUTLIER_REPLACE = 3,
       K_STUDENT_T3 = 4, K_UNIFORM = 5 };

typedef struct {
    int kind;
    uint64_t seed, tid;
    double std, p1, p2;
    int64_t offset;  /* first element index of the slice */
    float* out;
    int64_t begin, end; /* slice-relative range of this worker */
} job_t;

static void fill_range(const job_t* j) {
    int64_t e = j->offset + j->begin;
    const int64_t e_end = j->offset + j->end;
    while (e < e_end) {
        const uint64_t block = (uint64_t)e >> 2;
        double z[4], a[4], b[4], c[4], mu[4];
        switch (j->kind) {
        case K_NORMAL:
        case K_HALF_NORMAL:
            normal4(j->seed, j->tid, SUB_MAIN, block, z);
            break;
        case K_OUTLIER_SCALED:
            normal4(j->seed, j->tid, SUB_MAIN, block, z);
            uniform4(j->seed, j->tid, SUB_MASK, block, mu);
            break;
        case K_OUTLIER_REPLACE:
            normal4(j->seed, j->tid, SUB_MAIN, block, z);
            uniform4(j->seed, j->tid, SUB_MASK, block, mu);
            normal4(j->seed, j->tid, SUB_REPL, block, a);
            break;
        case K_STUDENT_T3:
            normal4(j->seed, j->tid, SUB_MAIN, block, z);
            normal4(j->seed, j->tid, SUB_CHI1, block, a);
            normal4(j->seed, j->tid, SUB_CHI2, block, b);
            normal4(j->seed, j->tid, SUB_CHI3, block, c);
            break;
        case K_UNIFORM:
            uniform4(j->seed, j->tid, SUB_MAIN, block, mu);
            break;
        default:
            return;
        }
        for (int w = (int)(e & 3); w < 4 && e < e_end; ++w, ++e) {
            double x;
            switch (j->kind) {
            case K_NORMAL: x = j->std * z[w]; break;
            case K_HALF_NORMAL: x = fabs(j->std * z[w]); break;
            case K_OUTLIER_SCALED:
                x = j->std * z[w];
                if (mu[w] < j->p1) x = x * j->p2;
                break;
            case K_OUTLIER_REPLACE:
                x = (mu[w] < j->p1) ? j->p2 * a[w] : j->std * z[w];
                break;
            case K_STUDENT_T3:
                x = j->std * z[w] / sqrt((a[w] * a[w] + b[w] * b[w] + c[w] * c[w]) / 3.0);
                break;
            case K_UNIFORM: x = j->std * (2.0 * mu[w] - 1.0); break;
            default: x = 0.0;
            }
            j->out[e - j->offset] = (float)x;
        }
    }
}

static void* worker(void* arg) {
    fill_range((const job_t*)arg);
    return NULL;
}

/* Fill out[0..n) with elements [offset, offset+n) of the stream.  Returns 0 on
 * success, -1 on a bad argument.  The result does not depend on `threads`. */
int synth_fill(int kind, uint64_t seed, uint64_t tid, double std, double p1, double p2,
               int64_t offset, int64_t n, float* out, int threads) {
    if (n < 0 || offset < 0 || (n > 0 && out == NULL) || kind < 0 || kind > K_UNIFORM) return -1;
    if (n == 0) return 0;
    if (threads < 1) threads = 1;
    if (threads > 64) threads = 64;
    if (n < (int64_t)1 << 16) threads = 1;
    job_t jobs[64];
    pthread_t th[64];
    const int64_t chunk = ((n + threads - 1) / threads + 3) & ~(int64_t)3;
    int started = 0;
    for (int t = 0; t < threads; ++t) {
        int64_t b = (int64_t)t * chunk, e = b + chunk;
        if (b >= n) break;
        if (e > n) e = n;
        jobs[t] = (job_t){kind, seed, tid, std, p1, p2, offset, out, b, e};
        ++started;
    }
    if (started == 1) {
        fill_range(&jobs[0]);
        return 0;
    }
    int launched = 0;
    for (int t = 0; t < started; ++t) {
        if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) break;
        ++launched;
    }
    for (int t = launched; t < started; ++t) fill_range(&jobs[t]);
    for (int t = 0; t < launched; ++t) pthread_join(th[t], NULL);
    return 0;
}
