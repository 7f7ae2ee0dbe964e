/* Plain C oracle for the data-movement results, for timing the CPU baseline.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite and by the CPU-baseline
 * leg of the benchmark, never by the product.  Naive scalar loops, no
 * blocking, no intrinsics; the only parallelism is a split of the outer loop
 * over threads.
 *
 * Pages:
 *   "CuTe Swizzle 学习手册", swizzle formula (the XOR of the B-bit field at
 *   bit M+S into the field at bit M).
 *   "CUDA 013 - Swizzle 的工作原理", problem statement (a row-major matrix
 *   written out column-major, i.e. dst[c][r] = src[r][c]).
 *   "cutlass 入门", the operand read that hands each thread of a matrix
 *   instruction its fragment: here lane l of a 16x32 block holds row l % 16
 *   and k = 8 * (l / 16) .. +7.
 */
#include <pthread.h>
#include <stdint.h>
#include <string.h>

/* S >= 0: the field at M+S is XORed into the field at M; S < 0: the field
 * at M is XORed into the field at M+|S| ("NVIDIA CuTe Swizzle", SShift). */
uint32_t oref_swizzle(uint32_t x, int32_t B, int32_t M, int32_t S) {
    int32_t src = S >= 0 ? M + S : M;
    int32_t dst = S >= 0 ? M : M - S;
    uint32_t yy = (x >> src) & ((1u << B) - 1u);
    return x ^ (yy << dst);
}

void oref_swizzle_map(const int32_t* in, int32_t* out, int64_t n, int32_t B, int32_t M, int32_t S) {
    for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)oref_swizzle((uint32_t)in[i], B, M, S);
}

/* ---- dst[b][c][r] = src[b][r][c], element size 1, 2 or 4 bytes ---- */
struct tr_job {
    const uint8_t* src;
    uint8_t* dst;
    int64_t rows, cols, first, last; /* flat (b, r) range */
    int32_t esz;
};

static void* tr_run(void* arg) {
    const struct tr_job* j = (const struct tr_job*)arg;
    for (int64_t br = j->first; br < j->last; ++br) {
        int64_t b = br / j->rows, r = br % j->rows;
        for (int64_t c = 0; c < j->cols; ++c) {
            int64_t s = (b * j->rows + r) * j->cols + c;
            int64_t d = (b * j->cols + c) * j->rows + r;
            memcpy(j->dst + d * j->esz, j->src + s * j->esz, (size_t)j->esz);
        }
    }
    return 0;
}

/* ---- frag[i][kb][l][e] = X[16 i + l % 16][32 kb + 8 (l / 16) + e] ---- */
struct st_job {
    const uint16_t* src;
    uint16_t* frag;
    int64_t k, first, last; /* range of i (16-row blocks) */
};

static void* st_run(void* arg) {
    const struct st_job* j = (const struct st_job*)arg;
    const int64_t kb_n = j->k / 32;
    for (int64_t i = j->first; i < j->last; ++i)
        for (int64_t kb = 0; kb < kb_n; ++kb)
            for (int l = 0; l < 64; ++l)
                for (int e = 0; e < 8; ++e)
                    j->frag[((i * kb_n + kb) * 64 + l) * 8 + e] = j->src[(16 * i + l % 16) * j->k + 32 * kb + 8 * (l / 16) + e];
    return 0;
}

#define OREF_MAX_THREADS 256

/* Returns 0, or -1 for a bad argument. */
int oref_convert(const void* src, void* dst, int64_t batch, int64_t rows, int64_t cols, int32_t esz, int32_t nthreads) {
    if ((esz != 1 && esz != 2 && esz != 4) || batch < 0 || rows < 0 || cols < 0 || nthreads < 1 || nthreads > OREF_MAX_THREADS) return -1;
    pthread_t th[OREF_MAX_THREADS];
    int started[OREF_MAX_THREADS] = {0};
    struct tr_job jobs[OREF_MAX_THREADS];
    const int64_t total = batch * rows;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (struct tr_job){(const uint8_t*)src, (uint8_t*)dst, rows, cols, total * t / nthreads, total * (t + 1) / nthreads, esz};
        if (t) started[t] = pthread_create(&th[t], 0, tr_run, &jobs[t]) == 0;
    }
    for (int t = 0; t < nthreads; ++t)
        if (!started[t]) tr_run(&jobs[t]); /* thread 0, and any thread that failed to start */
    for (int t = 1; t < nthreads; ++t)
        if (started[t]) pthread_join(th[t], 0);
    return 0;
}

int oref_stage_operand(const uint16_t* src, uint16_t* frag, int64_t mn, int64_t k, int32_t nthreads) {
    if (mn < 0 || k < 0 || mn % 16 || k % 32 || nthreads < 1 || nthreads > OREF_MAX_THREADS) return -1;
    pthread_t th[OREF_MAX_THREADS];
    int started[OREF_MAX_THREADS] = {0};
    struct st_job jobs[OREF_MAX_THREADS];
    const int64_t blocks = mn / 16;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (struct st_job){src, frag, k, blocks * t / nthreads, blocks * (t + 1) / nthreads};
        if (t) started[t] = pthread_create(&th[t], 0, st_run, &jobs[t]) == 0;
    }
    for (int t = 0; t < nthreads; ++t)
        if (!started[t]) st_run(&jobs[t]);
    for (int t = 1; t < nthreads; ++t)
        if (started[t]) pthread_join(th[t], 0);
    return 0;
}
