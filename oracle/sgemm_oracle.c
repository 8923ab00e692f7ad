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
 * oracle_sgemm_op also takes either operand transposed in storage (the
 * "GEneral" matrix-multiply of the BLAS, which the pages name but only use
 * untransposed): op(A)(i,k) = A[k*lda + i] when trans_a, op(B)(k,j) =
 * B[j*ldb + k] when trans_b.  The arithmetic is the same in every case.
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
 *
 * Two extensions for the workloads the pages name next to the GEMM ("The GEMM
 * Scrapbook", introduction: attention projections and the two GEMMs of a
 * feed-forward block), each the plain definition written out:
 *   - oracle_sgemm_strided_batched: `batch` independent products, operand b at
 *     A + b*stride_a, B + b*stride_b, C + b*stride_c (a stride of 0 shares
 *     one A or B across the batch); batch 0 touches nothing.
 *   - oracle_sgemm_epilogue: C = act(alpha * op(A) op(B) + beta * C + bias),
 *     bias[j] added to every cell of column j (the bias of a linear layer
 *     over its output features), act applied in double to the finished sum,
 *     then one rounding to float.  The pages name no activation; the codes
 *     are: 0 none, 1 ReLU max(x, 0), 2 SiLU x / (1 + e^-x) (Elfwing et al.,
 *     "Sigmoid-weighted linear units", 2018), 3 GELU x * Phi(x), Phi the
 *     standard normal CDF, 4 GELU's tanh approximation
 *     x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (both from Hendrycks
 *     and Gimpel, "Gaussian error linear units", 2016).  Phi(x) is evaluated
 *     as erfc(-x / sqrt 2) / 2 and (1 + tanh u) / 2 as 1 / (1 + e^(-2u)),
 *     identities that avoid the cancellation of 1 + erf and 1 + tanh for
 *     negative x.  With alpha == 0 or K == 0 the sum is beta * C + bias (A
 *     and B not read).
 *   - oracle_gemm_mixed: the same product with A and B given as 16-bit
 *     floats (bfloat16: the high half of an IEEE binary32; float16: IEEE
 *     binary16), C and the scalars in fp32 -- the reduced-precision inputs of
 *     the tensor-core hardware the fine print of "The GEMM Scrapbook" points
 *     to (fp16 rates above the fp32 ladder).  Every 16-bit value is decoded exactly
 *     (both formats embed in binary32) and the product is the definition
 *     above on the decoded values.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <stddef.h>

#define ORACLE_VERSION 4

/* activation codes of oracle_sgemm_epilogue */
#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_SILU 2
#define ORACLE_ACT_GELU_ERF 3
#define ORACLE_ACT_GELU_TANH 4

typedef struct {
    int i0, i1;          /* band of rows [i0, i1) */
    int N, K;
    double alpha, beta;
    const float *A; long long a_row, a_col;   /* op(A)(i,k) = A[i*a_row + k*a_col] */
    const float *B; long long b_row, b_col;   /* op(B)(k,j) = B[k*b_row + j*b_col] */
    float *C;       long long ldc;
    const float *bias;   /* per column of C, or NULL */
    int act;             /* ORACLE_ACT_* */
    int status;
} band_t;

/* The activation of the finished sum, in double. */
static double activate(int act, double x)
{
    switch (act) {
    case ORACLE_ACT_RELU: return x < 0.0 ? 0.0 : x;
    case ORACLE_ACT_SILU: return x / (1.0 + exp(-x));
    case ORACLE_ACT_GELU_ERF: return 0.5 * x * erfc(-x / sqrt(2.0));
    case ORACLE_ACT_GELU_TANH: {
        const double pi = 3.14159265358979323846;
        const double u = sqrt(2.0 / pi) * (x + 0.044715 * x * x * x);
        return x / (1.0 + exp(-2.0 * u));
    }
    default: return x;
    }
}

/* The epilogue of one cell: bias and activation of the finished sum. */
static float finish(const band_t *b, int j, double out)
{
    if (b->bias) out += (double)b->bias[j];
    return (float)activate(b->act, out);
}

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
                crow[j] = finish(b, j, (b->beta == 0.0) ? 0.0 : b->beta * (double)crow[j]);
            continue;
        }
        for (int j = 0; j < N; ++j) acc[j] = 0.0;
        const float *arow = b->A + (long long)i * b->a_row;
        for (int k = 0; k < K; ++k) {
            const double a = (double)arow[(long long)k * b->a_col];
            const float *brow = b->B + (long long)k * b->b_row;
            for (int j = 0; j < N; ++j)
                acc[j] += a * (double)brow[(long long)j * b->b_col];
        }
        for (int j = 0; j < N; ++j) {
            double out = b->alpha * acc[j];
            if (b->beta != 0.0)
                out += b->beta * (double)crow[j];
            crow[j] = finish(b, j, out);
        }
    }
    free(acc);
    b->status = 0;
    return NULL;
}

int oracle_version(void) { return ORACLE_VERSION; }

/*
 * Argument checks of oracle_sgemm_op, numbered in its parameter list:
 * 0 when every argument is valid.
 */
static int check_op(int trans_a, int trans_b, int M, int N, int K, float alpha,
                    const float *A, int lda, const float *B, int ldb, const float *C, int ldc)
{
    if (trans_a != 0 && trans_a != 1) return -1;
    if (trans_b != 0 && trans_b != 1) return -2;
    if (M < 0) return -3;
    if (N < 0) return -4;
    if (K < 0) return -5;
    const int a_cols = trans_a ? M : K, b_cols = trans_b ? K : N;
    if (lda < (a_cols > 1 ? a_cols : 1)) return -8;
    if (ldb < (b_cols > 1 ? b_cols : 1)) return -10;
    if (ldc < (N > 1 ? N : 1)) return -13;
    if (M == 0 || N == 0) return 0;
    const int reads_ab = (alpha != 0.0f && K > 0);
    if (reads_ab && !A) return -7;
    if (reads_ab && !B) return -9;
    if (!C) return -12;
    return 0;
}

/* One product over valid arguments (checked by the caller). */
static int sgemm_core(int trans_a, int trans_b, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb,
                      float beta, float *C, int ldc, const float *bias, int act, int nthreads)
{
    if (M == 0 || N == 0) return 0;
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
        b->A = A; b->a_row = trans_a ? 1 : lda; b->a_col = trans_a ? lda : 1;
        b->B = B; b->b_row = trans_b ? 1 : ldb; b->b_col = trans_b ? ldb : 1;
        b->C = C; b->ldc = ldc;
        b->bias = bias; b->act = act;
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

/*
 * C = alpha * op(A) * op(B) + beta * C with op(A) M x K and op(B) K x N.
 * Returns 0 on success; -i when the i-th argument is invalid (1-based, in the
 * order of the parameter list); -100 when memory for the row accumulators or
 * threads could not be obtained.  nthreads <= 0 means one thread.
 */
int oracle_sgemm_op(int trans_a, int trans_b, int M, int N, int K, float alpha,
                    const float *A, int lda, const float *B, int ldb,
                    float beta, float *C, int ldc, int nthreads)
{
    const int st = check_op(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (st != 0) return st;
    return sgemm_core(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, NULL,
                      ORACLE_ACT_NONE, nthreads);
}

/*
 * C = act(alpha * op(A) * op(B) + beta * C + bias): oracle_sgemm_op's
 * arguments, then bias (N floats, one per column of C; NULL for none) and act
 * (an ORACLE_ACT_* code).  Returns as oracle_sgemm_op, and -15 for an unknown
 * act.
 */
int oracle_sgemm_epilogue(int trans_a, int trans_b, int M, int N, int K, float alpha,
                          const float *A, int lda, const float *B, int ldb,
                          float beta, float *C, int ldc, const float *bias, int act,
                          int nthreads)
{
    const int st = check_op(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (st != 0) return st;
    if (act < ORACLE_ACT_NONE || act > ORACLE_ACT_GELU_TANH) return -15;
    return sgemm_core(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, bias, act,
                      nthreads);
}

/*
 * `batch` products C_b = alpha * op(A_b) * op(B_b) + beta * C_b, with
 * A_b = A + b*stride_a, B_b = B + b*stride_b, C_b = C + b*stride_c (floats).
 * Arguments, 1-based: trans_a, trans_b, M, N, K, alpha, A, lda, stride_a, B,
 * ldb, stride_b, beta, C, ldc, stride_c, batch, nthreads.  Returns 0, or -i
 * for an invalid i-th argument: a negative stride of A or B, a stride of C
 * that lets two of the batch's C matrices overlap (stride_c < (M-1)*ldc + N
 * with batch > 1), a negative batch, or any check of oracle_sgemm_op.
 */
int oracle_sgemm_strided_batched(int trans_a, int trans_b, int M, int N, int K, float alpha,
                                 const float *A, int lda, long long stride_a,
                                 const float *B, int ldb, long long stride_b,
                                 float beta, float *C, int ldc, long long stride_c,
                                 int batch, int nthreads)
{
    static const int renumber[14] = {0, -1, -2, -3, -4, -5, -6, -7, -8, -10, -11, 0, -14, -15};
    const int st = check_op(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (st != 0) return renumber[-st];
    if (stride_a < 0) return -9;
    if (stride_b < 0) return -12;
    if (batch < 0) return -17;
    if (batch > 1 && M > 0 && N > 0 && stride_c < (long long)(M - 1) * ldc + N) return -16;
    for (int b = 0; b < batch; ++b) {
        const int r = sgemm_core(trans_a, trans_b, M, N, K, alpha, A ? A + b * stride_a : A, lda,
                                 B ? B + b * stride_b : B, ldb, beta, C + b * stride_c, ldc, NULL,
                                 ORACLE_ACT_NONE, nthreads);
        if (r != 0) return r;
    }
    return 0;
}

/* 16-bit input formats of oracle_gemm_mixed */
#define ORACLE_BF16 1
#define ORACLE_F16 2

/* The exact value of a 16-bit float. */
static float decode16(int dtype, uint16_t h)
{
    if (dtype == ORACLE_BF16) {
        /* the high 16 bits of a binary32 (sign, 8-bit exponent, 7 stored
           fraction bits); the low half is zero */
        const uint32_t bits = (uint32_t)h << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    /* binary16: sign, 5-bit exponent (bias 15), 10 fraction bits */
    const int sign = (h >> 15) & 1, e = (h >> 10) & 31, frac = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)frac, -24);                   /* zero and subnormals */
    else if (e == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), e - 25);       /* 1.frac x 2^(e-15) */
    return (float)(sign ? -v : v);
}

/*
 * C = alpha * op(A) * op(B) + beta * C with A and B stored as 16-bit floats
 * (dtype ORACLE_BF16 or ORACLE_F16; storage and leading dimensions in
 * elements as oracle_sgemm_op's) and C in fp32.  Arguments: dtype, then
 * oracle_sgemm_op's.  Returns 0, -1 for an unknown dtype, or oracle_sgemm_op's
 * codes shifted by one; -100 when memory is short.
 */
int oracle_gemm_mixed(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                      const uint16_t *A, int lda, const uint16_t *B, int ldb,
                      float beta, float *C, int ldc, int nthreads)
{
    if (dtype != ORACLE_BF16 && dtype != ORACLE_F16) return -1;
    /* the checks look at the arguments only, not at the data */
    const int st = check_op(trans_a, trans_b, M, N, K, alpha, (const float *)A, lda,
                            (const float *)B, ldb, C, ldc);
    if (st != 0) return st - 1;
    if (M == 0 || N == 0) return 0;
    const int reads_ab = (alpha != 0.0f && K > 0);
    const long long a_rows = trans_a ? K : M, b_rows = trans_b ? N : K;
    const long long a_cols = trans_a ? M : K, b_cols = trans_b ? K : N;
    float *a = NULL, *b = NULL;
    if (reads_ab) {
        a = (float *)malloc(sizeof(float) * (size_t)(a_rows * a_cols));
        b = (float *)malloc(sizeof(float) * (size_t)(b_rows * b_cols));
        if (!a || !b) { free(a); free(b); return -100; }
        for (long long r = 0; r < a_rows; ++r)
            for (long long c = 0; c < a_cols; ++c)
                a[r * a_cols + c] = decode16(dtype, A[r * lda + c]);
        for (long long r = 0; r < b_rows; ++r)
            for (long long c = 0; c < b_cols; ++c)
                b[r * b_cols + c] = decode16(dtype, B[r * ldb + c]);
    }
    const int r = sgemm_core(trans_a, trans_b, M, N, K, alpha, a, (int)(a_cols > 1 ? a_cols : 1),
                             b, (int)(b_cols > 1 ? b_cols : 1), beta, C, ldc, NULL,
                             ORACLE_ACT_NONE, nthreads);
    free(a);
    free(b);
    return r;
}

/* The untransposed product, with the argument numbering of its own list. */
int oracle_sgemm(int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb,
                 float beta, float *C, int ldc, int nthreads)
{
    const int st = oracle_sgemm_op(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nthreads);
    return st < 0 && st > -100 ? st + 2 : st;   /* drop the two leading trans arguments */
}
