/*
 * fp32_sgemm.h -- C ABI of the MI355X (gfx950) single-precision GEMM library.
 *
 * Operation (the one every entry point computes):
 *     C = alpha * (A * B) + beta * C
 * with A of size M x K, B of size K x N and C of size M x N, all fp32; every
 * cell of C is the dot product of one row of A and one column of B.
 *   -- "a CUDA matmul" (plasmient.com labs), section 00 "Start here": the
 *      SGEMM definition and its alpha/beta form; section 02: the kernel
 *      signature (M, N, K, alpha, A, B, beta, C) this ABI extends.
 *   -- "The GEMM Scrapbook" (iamartyaa.github.io), introduction: A is M x K,
 *      B is K x N, C is M x N, each cell a row-by-column dot product.
 *   -- "The 1% kernel" (notes.ybc.sh, GPU level 1), section 4: row-major
 *      flat storage, element (r, c) at offset r * width + c.
 *
 * Layout: row-major with leading dimensions (counted in floats):
 *     A(i,k) = A[i*lda + k],  B(k,j) = B[k*ldb + j],  C(i,j) = C[i*ldc + j]
 * Requirements: lda >= max(1,K), ldb >= max(1,N), ldc >= max(1,N).  Floats of
 * a row beyond its logical width (the padding) are never read, and never
 * written in C.
 *
 * Memory and ownership: A, B and C are DEVICE pointers owned by the caller.
 * The library keeps no pointer to them after a call returns.  It allocates
 * device memory in two cases only, both for partial sums: a stream-K launch
 * (SGEMM_FLAG_STREAMK, or chosen by automatic dispatch for a single product
 * with few tiles of C and a long K, whose last wave of workgroups would be
 * partly idle; two tile accumulators for each of 256 workgroups: 64 MiB with
 * 256 x 128 tiles, 128 MiB with 256 x 256), and a few-rows skinny launch split
 * over K (automatic dispatch splits single products of M <= 16 rows whose
 * column strips leave most CUs idle, e.g. 1 x 4096 x 4096; a slice count
 * times M x N floats).  The workspace also holds 16 KiB of arrival counters.
 * Outside graph capture it is kept per device and stream and reused by later
 * calls on that stream (taken with hipMallocAsync on the stream, grown when a
 * call needs more, the old buffer returned with hipFreeAsync on the same
 * stream; held until sgemm_workspace_release or process exit; the per-thread
 * default stream gets one per host thread).  Under graph capture each call
 * records its own allocation and free on the capturing stream.  An
 * allocation failure is returned as its hipError_t.  Callers that cannot
 * allocate use sgemm_op_ex_noalloc.  Work is
 * enqueued on `stream` (NULL = the null stream) and the call
 * returns without synchronising: the caller keeps A, B and C alive and
 * unmodified until that stream's work has completed.  C must not overlap A
 * or B (A and B may alias each other).  Calls are thread-safe.
 *
 * Special cases (the pages are silent; these follow the reference BLAS):
 *   - M == 0 or N == 0: nothing is done.
 *   - alpha == 0 or K == 0: C = beta * C; A and B are not read.  With
 *     beta == 1 as well, nothing is done.
 *   - beta == 0: C is written without being read, so NaN/Inf already in C
 *     never reaches the result.
 *
 * Status codes returned by every compute entry point:
 *     0                 success (work enqueued)
 *     -i (1..12)        the i-th argument is invalid (1-based, in the order
 *                       of sgemm's parameter list): a negative dimension, a
 *                       leading dimension that is too small, a null pointer
 *                       for an operand that will be read or written, or a
 *                       pointer that is not 4-byte aligned
 *     -13               sgemm_ex: the configuration is invalid or does not
 *                       apply to this shape (see sgemm_config); sgemm_op:
 *                       no compiled kernel serves this transposition
 *     -21, -22          sgemm_op: trans_a, trans_b not 0 or 1 (sgemm_cblas:
 *                       not 111, 112 or 113)
 *     -23               sgemm_cblas: order not 101 or 102
 *     -24, -25          sgemm_epilogue: bias not 4-byte aligned; unknown act
 *     -26, -27, -28     sgemm_strided_batched: negative stride of A or B; a
 *                       stride of C that lets two of the batch's C overlap
 *     -29               sgemm_strided_batched: negative batch
 *     -30               sgemm_mixed: dtype not SGEMM_DTYPE_BF16 / _F16
 *     -31               sgemm_op_ex_noalloc: the plan's partial sums need
 *                       more memory than the static scratch holds
 *     > 0               a hipError_t reported by the kernel launch
 * No C++ exception crosses this interface.
 *
 * Numerics: products are accumulated in fp32 (fp32 MFMA or fp32 FMA); the
 * order of the K-sum is implementation-defined but fixed for a given shape and
 * configuration, so repeated calls give bitwise-identical results.  No input
 * is rounded to a narrower format.
 */
#ifndef FP32_SGEMM_H
#define FP32_SGEMM_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

/* Kernel families selectable through sgemm_config.variant. */
enum sgemm_variant {
    SGEMM_VARIANT_AUTO = 0,    /* choose by shape (what sgemm() does) */
    SGEMM_VARIANT_MFMA = 1,    /* fp32 matrix-core (v_mfma_f32_*_f32) tiles */
    SGEMM_VARIANT_VALU = 2,    /* per-thread register micro-tiles of fp32 FMAs */
    SGEMM_VARIANT_SKINNY = 3,  /* memory-bound shapes: M <= 16 or N <= 16 */
    SGEMM_VARIANT_MFMA16 = 4,  /* sgemm_mixed: 16-bit-input matrix-core tiles */
    SGEMM_VARIANT_GENERIC16 = 5, /* sgemm_mixed: the generic 16-bit-input kernel */
    SGEMM_VARIANT_SMALL = 6,   /* small products: one wave per 16 x 16 or 16 x 64 block of C,
                                  operands from memory into registers, optional k-groups;
                                  A untransposed (either B) */
    SGEMM_VARIANT_COUNT = 7
};

/* Input formats of sgemm_mixed. */
#define SGEMM_DTYPE_BF16 1   /* bfloat16: the high 16 bits of an IEEE binary32 */
#define SGEMM_DTYPE_F16 2    /* IEEE binary16 */

/* sgemm_config.flags bits */
#define SGEMM_FLAG_SCALAR_IO 0x1   /* force 4-byte loads/stores (no 16-byte vectors) */
#define SGEMM_FLAG_UNTUNED 0x2     /* automatic choice: skip the tuned table, use the cost model */
#define SGEMM_FLAG_STREAMK 0x4     /* with an explicit MFMA tile that offers it: stream-K
                                      (see sgemm_ex); reported by sgemm_plan when chosen */

/*
 * Explicit configuration for sgemm_ex: which kernel family, which compiled
 * tile configuration of that family (`tile` indexes the list reported by
 * sgemm_tile_info; -1 = the family's choice for the shape), and flag bits.
 * `group_m` sets the number of tile-rows per block of the tile-ordering
 * swizzle (0 = the library's choice).  For the few-rows tiles of the skinny
 * family it is instead the number of K slices to split a single product
 * over (at most 64, and at most one per 16-row k-chunk of each wave; 1 = no
 * split; 0 = the library's choice; batches are not split).
 */
typedef struct sgemm_config {
    int variant;
    int tile;
    int flags;
    int group_m;
} sgemm_config;

/* Description of one compiled tile configuration. */
typedef struct sgemm_tile_desc {
    int bm, bn, bk;   /* workgroup tile of C (bm x bn) and K step (bk) */
    int wm, wn;       /* per-wave tile of C */
    int tm, tn;       /* per-lane micro-tile (VALU family; 0 for MFMA); skinny family:
                         tm = kernel kind (0: few rows of C, 1: few columns); small
                         family: tm = k-groups (waves sharing one block of C over K) */
    int threads;      /* workgroup size */
    int lds_bytes;    /* LDS per workgroup */
    int stages;       /* LDS buffers in the K pipeline (0: no LDS staging) */
    int flags;        /* SGEMM_TILE_* bits */
} sgemm_tile_desc;

/* sgemm_tile_desc.flags: the tile only serves problems made of whole tiles
 * (M, N, K multiples of bm, bn, bk) with A, B, C 16-byte aligned, leading
 * dimensions that are multiples of 4, and bm * lda and bk * ldb below 2^29
 * elements (31-bit byte offsets within one tile's panel).  Asked for explicitly
 * elsewhere, sgemm_ex returns -13; automatic dispatch never picks it there. */
#define SGEMM_TILE_WHOLE 0x1
/* sgemm_tile_desc.flags: the tile's loads go straight from memory to LDS
 * through 32-bit buffer offsets, so it needs bm * lda and bk * ldb below 2^29
 * elements; sgemm_ex returns -13 otherwise. */
#define SGEMM_TILE_DIRECT 0x2
/* sgemm_tile_desc.flags: the tile also serves B stored transposed
 * (sgemm_op with trans_b = 1). */
#define SGEMM_TILE_TRANS_B 0x4
/* sgemm_tile_desc.flags: the tile serves A stored transposed (sgemm_op with
 * trans_a = 1), and only that; such tiles need bk * lda below 2^29 elements. */
#define SGEMM_TILE_TRANS_A 0x8
/* sgemm_tile_desc.flags: the tile can also run as stream-K: 256 persistent
 * workgroups take the tiles of the last one or two waves (whole waves before
 * them run as usual) as one list of k-steps cut into 256 equal runs; a run
 * that ends or starts inside a tile leaves that tile's partial sums in a
 * workspace, and a second launch adds each tile's pieces in k order and
 * applies alpha, beta and C.  A batch (sgemm_strided_batched) runs the same
 * persistent workgroups over the whole tiles of all its entries, with no
 * split and no workspace.  Offered where A and B take 16-byte loads (rows
 * 16-byte aligned, the stored row length a multiple of 4); asked for with
 * SGEMM_FLAG_STREAMK, otherwise sgemm_ex returns -13.  The k-sum order then
 * depends on the split, which is fixed for a shape: results stay bitwise
 * repeatable. */
#define SGEMM_TILE_STREAMK 0x10

/*
 * sgemm: C = alpha * (A * B) + beta * C, kernel family and tile chosen from
 * the shape.  Arguments, in order: M, N, K (dimensions, >= 0); alpha; A
 * (device, M x K, leading dimension lda); B (device, K x N, ldb); beta; C
 * (device, M x N, ldc, read when beta != 0 and written); stream.
 * Returns a status code as described above.
 */
int sgemm(int M, int N, int K, float alpha,
          const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, hipStream_t stream);

/*
 * sgemm_ex: as sgemm, with the kernel family and tile taken from *cfg
 * (NULL = automatic, identical to sgemm).  Returns -13 when cfg names an
 * unknown family or tile index, or a family that does not apply to the shape
 * (SGEMM_VARIANT_SKINNY requires M <= 16 or N <= 16), or SGEMM_FLAG_STREAMK
 * without an MFMA tile flagged SGEMM_TILE_STREAMK, with SGEMM_FLAG_SCALAR_IO,
 * or for operands stream-K does not take.  Used by the tuner, the benchmark
 * and the tests to reach each family directly.
 */
int sgemm_ex(int M, int N, int K, float alpha,
             const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, hipStream_t stream,
             const sgemm_config *cfg);

/*
 * sgemm_select: the configuration sgemm() would use for this shape and these
 * pointers/leading dimensions, written to *out (variant, tile, flags,
 * group_m; for a few-rows skinny tile, group_m is the number of K slices the
 * product is split into, 1 for none, so that *out passed to sgemm_ex runs
 * the same plan).  When sgemm() also hands edge strips to the skinny family (see
 * sgemm_plan), *out describes the main part.  Reads no memory behind A, B or
 * C.  Returns 0; -1, -2 or -3 for a negative M, N or K; -14 when out is NULL.
 */
int sgemm_select(int M, int N, int K, const float *A, int lda, const float *B,
                 int ldb, const float *C, int ldc, sgemm_config *out);

/*
 * sgemm_op: C = alpha * op(A) * op(B) + beta * C, the general form of the
 * BLAS (row-major, as cblas_sgemm with CblasRowMajor).  op(A) is M x K:
 * A itself (trans_a = 0, stored M x K, lda >= max(1, K)) or A transposed
 * (trans_a = 1, stored K x M, lda >= max(1, M)).  op(B) is K x N: B
 * (trans_b = 0, stored K x N, ldb >= max(1, N)) or B transposed (trans_b = 1,
 * stored N x K, ldb >= max(1, K): a weight matrix of a linear layer, C = X W^T).
 * Status codes as sgemm's for the arguments they share (-1 M .. -11 ldc),
 * -21 / -22 for a trans flag other than 0 or 1, and -13 when no compiled
 * kernel serves the transposition.  Transposed operands are served by the
 * MFMA family's direct-load tiles: trans_a = 0 with trans_b = 1 by those
 * flagged SGEMM_TILE_TRANS_B, trans_a = 1 (either trans_b) by those flagged
 * SGEMM_TILE_TRANS_A.  sgemm_op(0, 0, ...) is sgemm.
 */
int sgemm_op(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
             int lda, const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream);

/* sgemm_op with an explicit configuration, as sgemm_ex (MFMA family only when
 * an operand is transposed). */
int sgemm_op_ex(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                int lda, const float *B, int ldb, float beta, float *C, int ldc,
                hipStream_t stream, const sgemm_config *cfg);

/*
 * sgemm_op_ex_noalloc: sgemm_op_ex for callers that cannot allocate device
 * memory -- code under HIP graph capture (where sgemm_op would record an
 * allocation and a free node for every split or stream-K call), tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no hipMalloc, hipFree or
 * allocating routine: the partial sums of split launches go to a static
 * device array of the library (16 MiB plus 16 KiB of arrival counters), held
 * by every device the library runs on until the process ends.  Arguments,
 * results and status codes as sgemm_op_ex (cfg NULL = automatic); the
 * automatic plan is sgemm_op's among the plans whose partial sums fit the
 * array (stream-K, which needs 64 MiB or more, is then never chosen), and a
 * call whose explicit configuration needs more returns -31 before launching
 * anything.  Every call on a device shares that device's array: calls that
 * may overlap on one device (on different streams, or from several host
 * threads) race on it, and must be ordered by the caller.
 */
int sgemm_op_ex_noalloc(int trans_a, int trans_b, int M, int N, int K, float alpha,
                        const float *A, int lda, const float *B, int ldb, float beta, float *C,
                        int ldc, hipStream_t stream, const sgemm_config *cfg);

/*
 * Activation codes of sgemm_epilogue (applied in fp32 to the finished sum).
 * The pages name the feed-forward GEMMs of a transformer ("The GEMM
 * Scrapbook", introduction) but no activation; these are the common ones.
 */
#define SGEMM_ACT_NONE 0       /* x */
#define SGEMM_ACT_RELU 1       /* max(x, 0) */
#define SGEMM_ACT_SILU 2       /* x / (1 + exp(-x)) */
#define SGEMM_ACT_GELU_ERF 3   /* x * Phi(x), Phi the standard normal CDF */
#define SGEMM_ACT_GELU_TANH 4  /* x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */

/*
 * sgemm_epilogue: C = act(alpha * op(A) * op(B) + beta * C + bias), the
 * product of a linear layer with its bias and activation fused ("The GEMM
 * Scrapbook", introduction: the two GEMMs of a feed-forward block).
 * Arguments as sgemm_op, then bias (device, N floats: bias[j] is added to
 * every cell of column j; NULL for none), act (SGEMM_ACT_*) and the stream.
 * beta == 0 never reads C.  alpha == 0 or K == 0 gives act(beta * C + bias)
 * without reading A or B.  The direct-load MFMA tiles and the skinny family
 * apply bias and activation in their own epilogue when every operand allows
 * 16-byte I/O; otherwise the product is stored and one elementwise pass
 * applies them.  Status codes as sgemm_op's, -24 for a bias that is not
 * 4-byte aligned, -25 for an unknown act.
 */
int sgemm_epilogue(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                   int lda, const float *B, int ldb, float beta, float *C, int ldc,
                   const float *bias, int act, hipStream_t stream);

/* sgemm_epilogue with an explicit configuration, as sgemm_op_ex. */
int sgemm_epilogue_ex(int trans_a, int trans_b, int M, int N, int K, float alpha,
                      const float *A, int lda, const float *B, int ldb, float beta, float *C,
                      int ldc, const float *bias, int act, hipStream_t stream,
                      const sgemm_config *cfg);

/*
 * sgemm_strided_batched: `batch` independent products
 *     C_b = alpha * op(A_b) * op(B_b) + beta * C_b,  b = 0 .. batch-1,
 * with A_b = A + b * stride_a, B_b = B + b * stride_b, C_b = C + b * stride_c
 * (strides in floats; a stride of 0 for A or B shares that operand across
 * the batch, e.g. one weight matrix for many inputs).  Other arguments as
 * sgemm_op.  The C matrices must not overlap: stride_c >= (M-1)*ldc + N when
 * batch > 1 (-28 otherwise).  batch == 0 does nothing.  One kernel launch
 * serves up to 65535 entries (grid y), larger batches take several.  The
 * work of attention projections and heads ("The GEMM Scrapbook",
 * introduction).  Status codes as sgemm_op's, and -26 / -27 for a negative
 * stride of A / B, -29 for a negative batch.
 */
int sgemm_strided_batched(int trans_a, int trans_b, int M, int N, int K, float alpha,
                          const float *A, int lda, long long stride_a, const float *B, int ldb,
                          long long stride_b, float beta, float *C, int ldc, long long stride_c,
                          int batch, hipStream_t stream);

/* sgemm_strided_batched with an explicit configuration, as sgemm_op_ex. */
int sgemm_strided_batched_ex(int trans_a, int trans_b, int M, int N, int K, float alpha,
                             const float *A, int lda, long long stride_a, const float *B,
                             int ldb, long long stride_b, float beta, float *C, int ldc,
                             long long stride_c, int batch, hipStream_t stream,
                             const sgemm_config *cfg);

/*
 * sgemm_mixed: C = alpha * op(A) * op(B) + beta * C with A and B given as
 * 16-bit floats (dtype SGEMM_DTYPE_BF16 or SGEMM_DTYPE_F16; device arrays of
 * 16-bit values, leading dimensions in elements) and C, alpha, beta in fp32.
 * Every product of two 16-bit values is exact in fp32; sums are accumulated
 * in fp32 (the matrix instructions v_mfma_f32_16x16x32_bf16 / _f16).  The
 * reduced-precision matrix hardware of the tensor-core fine print of "The
 * GEMM Scrapbook".  Arguments after dtype as sgemm_op's.  The matrix-core
 * tiles (family SGEMM_VARIANT_MFMA16) serve trans_a = 0, trans_b = 1 (C = X
 * W^T with W stored N x K) when K, lda and ldb are even and A, B are 4-byte
 * aligned; automatic dispatch runs such products of at most 8 rows (16
 * where the rows of A and W take 16-byte loads) through the few-rows kernel
 * of the skinny family in the same word form, streaming W once; every other
 * case runs the generic kernel
 * (SGEMM_VARIANT_GENERIC16: 16-bit values decoded to fp32 in LDS, fp32
 * FMAs; correct for any layout, not tuned).  A and B need 2-byte alignment
 * (-5, -7).  Status codes as sgemm_op's, -30 for an unknown dtype, -13 when
 * an explicit configuration cannot serve the operands.
 */
int sgemm_mixed(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                const void *A, int lda, const void *B, int ldb, float beta, float *C, int ldc,
                hipStream_t stream);

/* sgemm_mixed with an explicit configuration (variant SGEMM_VARIANT_MFMA16
 * with a tile index, or SGEMM_VARIANT_GENERIC16 with tile 0 or -1). */
int sgemm_mixed_ex(int dtype, int trans_a, int trans_b, int M, int N, int K, float alpha,
                   const void *A, int lda, const void *B, int ldb, float beta, float *C, int ldc,
                   hipStream_t stream, const sgemm_config *cfg);

/*
 * sgemm_cblas: the same product with the argument conventions of
 * cblas_sgemm: order 101 (row-major) or 102 (column-major), trans_a and
 * trans_b 111 (no transpose), 112 (transpose) or 113 (conjugate transpose,
 * the same for real matrices), then M, N, K, alpha, A, lda, B, ldb, beta, C,
 * ldc and the stream.  Row-major calls are sgemm_op; a column-major call runs
 * as the row-major product C^T = op(B)^T op(A)^T over the same memory (no
 * copy).  Leading dimensions follow the order: column-major A (no transpose)
 * needs lda >= max(1, M), and so on.  Status codes as sgemm_op's, naming the
 * caller's arguments (-1 M, -2 N, -5 A, -6 lda, -7 B, -8 ldb, -21 trans_a,
 * -22 trans_b ...), and -23 for an order other than 101 or 102.
 */
int sgemm_cblas(int order, int trans_a, int trans_b, int M, int N, int K, float alpha,
                const float *A, int lda, const float *B, int ldb, float beta, float *C, int ldc,
                hipStream_t stream);

/*
 * sgemm_op_plan: sgemm_plan for sgemm_op's transposition flags (0 or 1; -21 /
 * -22 otherwise).  Transposed problems get no edge strips.
 */
int sgemm_op_plan(int trans_a, int trans_b, int M, int N, int K, const float *A, int lda,
                  const float *B, int ldb, const float *C, int ldc, sgemm_config *out,
                  int *edge_rows, int *edge_cols);

/*
 * sgemm_plan: sgemm_select plus the edge strips of the automatic plan.  When
 * the chosen MFMA tile would leave at most 16 rows (columns) in an extra,
 * mostly idle round of workgroups, sgemm() computes the last *edge_rows rows
 * (last *edge_cols columns) of C with the skinny family in a second (third)
 * launch on the same stream and the rest with the tile in *out.  edge_rows
 * and edge_cols may be NULL.  Same return values as sgemm_select.
 */
int sgemm_plan(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
               const float *C, int ldc, sgemm_config *out, int *edge_rows, int *edge_cols);

/* Number of compiled tile configurations of a family (0 for unknown). */
int sgemm_tile_count(int variant);

/* Describe tile configuration `tile` of `variant`; 0 on success, -13 if none. */
int sgemm_tile_info(int variant, int tile, sgemm_tile_desc *out);

/* Static text for a status code (never NULL). */
const char *sgemm_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int sgemm_version(void);

/*
 * sgemm_workspace_release: synchronise the current device and free the
 * workspaces the library keeps for it (one per stream that has run a
 * stream-K or split-K launch; see "Memory and ownership").  Later calls take
 * new ones as needed.  Returns 0 or a hipError_t.  Not to be called while
 * another thread runs sgemm calls on the same device.  Call it before
 * destroying a stream that has run such launches: a stream created later
 * may receive the same handle value and would otherwise inherit the buffer.
 */
int sgemm_workspace_release(void);

#ifdef __cplusplus
}
#endif

#endif /* FP32_SGEMM_H */
