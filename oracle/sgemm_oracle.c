/*
 * sgemm_oracle.c -- plain CPU reference for single-precision GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle against which
 * the GPU library is checked.  Only the test-suite, the smoke check and the
 * benchmark's cpu_baseline leg may load it.  It shares no code, header, build
 * flag or helper with the GPU library, and the GPU library never calls it.
 *
 * What it computes (the operation the pages define):
 *   C = alpha * (A * B) + beta * C, with A of size M x K, B of size K x N and
 *   C of size M x N, every cell of C being the dot product of one row of A
 *   with one column of B.
 *   -- "a CUDA matmul" (plasmient.com labs), section 00 "Start here"
 *   -- "The GEMM Scrapbook" (iamartyaa.github.io), introduction (GEMM, M x K
 *      times K x N, each cell a row-by-column dot product)
 *   -- "The 1% kernel" (notes.ybc.sh, GPU level 1), section 1 (the cell formula)
 *
 * Storage: row-major flat arrays ("The 1% kernel", section 4: element (r, c)
 * lives at offset r * width + c), generalised with leading dimensions:
 *   A(i,k) = A[i*lda + k],  B(k,j) = B[k*ldb + j],  C(i,j) = C[i*ldc + j].
 *
 * Arithmetic: every product of two floats is exact in double (24+24 <= 53
 * significant bits); the K products of a cell are summed in double in
 * ascending k; the epilogue alpha*acc (+ beta*C) is formed in double and
 * rounded to float once.
 *
 * Readings where the pages are silent (BLAS reference conventions):
 *   - M == 0 or N == 0: nothing is touched.
 *   - alpha == 0 or K == 0: C = beta * C; A and B are not read.
 *   - beta == 0: C is written without being read (so NaN/Inf already in C
 *     does not leak into the result).
 *
 * Loop form: i-k-j with a double row accumulator, so the innermost loop walks
 * a row of B.  Rows of C are split into contiguous bands, one POSIX thread per
 * band; each cell is produced by exactly one thread, in the same order, so the
 * result does not depend on the thread count.
 */
#include <pthread.h>
#include <stdlib.h>
#include <stddef.h>

#define ORACLE_VERSION 1

typedef struct {
    int i0, i1;          /* band of rows [i0, i1) */
    int N, K;
    double alpha, beta;
    const float *A; long long lda;
    const float *B; long long ldb;
    float *C;       long long ldc;
    int status;
} band_t;

/* C(i,:) for every i in the band. */
static void *run_band(void *arg)
{
    band_t *b = (band_t *)arg;
    const int N = b->N, K = b->K;
    double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    if (!acc) { b->status = -100; return NULL; }
    for (int i = b->i0; i < b->i1; ++i) {
        float *crow = b->C + (long long)i * b->ldc;
        if (b->alpha == 0.0 || K == 0) {
            /* C = beta * C; A and B are not read. */
            for (int j = 0; j < N; ++j)
                crow[j] = (b->beta == 0.0) ? 0.0f : (float)(b->beta * (double)crow[j]);
            continue;
        }
        for (int j = 0; j < N; ++j) acc[j] = 0.0;
        const float *arow = b->A + (long long)i * b->lda;
        for (int k = 0; k < K; ++k) {
            const double a = (double)arow[k];
            const float *brow = b->B + (long long)k * b->ldb;
            for (int j = 0; j < N; ++j)
                acc[j] += a * (double)brow[j];
        }
        for (int j = 0; j < N; ++j) {
            double out = b->alpha * acc[j];
            if (b->beta != 0.0)
                out += b->beta * (double)crow[j];
            crow[j] = (float)out;
        }
    }
    free(acc);
    b->status = 0;
    return NULL;
}

int oracle_version(void) { return ORACLE_VERSION; }

/*
 * Returns 0 on success; -i when the i-th argument is invalid (1-based, in the
 * order of the parameter list); -100 when memory for the row accumulators or
 * threads could not be obtained.  nthreads <= 0 means one thread.
 */
int oracle_sgemm(int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb,
                 float beta, float *C, int ldc, int nthreads)
{
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    if (lda < (K > 1 ? K : 1)) return -6;
    if (ldb < (N > 1 ? N : 1)) return -8;
    if (ldc < (N > 1 ? N : 1)) return -11;
    if (M == 0 || N == 0) return 0;
    const int reads_ab = (alpha != 0.0f && K > 0);
    if (reads_ab && !A) return -5;
    if (reads_ab && !B) return -7;
    if (!C) return -10;

    if (nthreads < 1) nthreads = 1;
    if (nthreads > M) nthreads = M;

    band_t *bands = (band_t *)calloc((size_t)nthreads, sizeof(band_t));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int *started = (int *)calloc((size_t)nthreads, sizeof(int));
    if (!bands || !tids || !started) { free(bands); free(tids); free(started); return -100; }

    for (int t = 0; t < nthreads; ++t) {
        band_t *b = &bands[t];
        b->i0 = (int)((long long)M * t / nthreads);
        b->i1 = (int)((long long)M * (t + 1) / nthreads);
        b->N = N; b->K = K;
        b->alpha = (double)alpha; b->beta = (double)beta;
        b->A = A; b->lda = lda; b->B = B; b->ldb = ldb; b->C = C; b->ldc = ldc;
        b->status = -100;
    }
    int status = 0;
    for (int t = 1; t < nthreads; ++t)
        started[t] = (pthread_create(&tids[t], NULL, run_band, &bands[t]) == 0);
    run_band(&bands[0]);
    for (int t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(tids[t], NULL);
        else run_band(&bands[t]);   /* thread could not start: do the band here */
    }
    for (int t = 0; t < nthreads; ++t)
        if (bands[t].status != 0) status = bands[t].status;
    free(bands); free(tids); free(started);
    return status;
}
