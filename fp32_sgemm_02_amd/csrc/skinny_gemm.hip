// skinny_gemm.hip -- SGEMM shapes with few rows (M <= 16) or few columns
// (N <= 16) of C.  They do O(1) flops per byte of the large operand, far below
// the ridge point of the roofline ("The GEMM Scrapbook", roofline paragraph:
// peak flops over memory bandwidth), so they are bound by HBM and the kernels
// are built to stream the large operand exactly once with wide, coalesced
// loads, with K split over the waves of a workgroup and a fixed-order LDS
// reduction (no atomics, so results are bitwise repeatable).
//
// Few rows (kind 0): C (M x N) = A (M x K) * B (K x N), B streamed.  The M <= 16
// rows of A are the A operand of v_mfma_f32_16x16x4_f32 (rows >= M read as
// zero); each workgroup owns a strip of 16*VW columns.  Lane l (i = l % 16,
// g = l / 16) in MFMA step s of a 16-wide k-chunk supplies k = 4g + s, and VW
// consecutive B values of row k (columns VW*i + c, c < VW, feed MFMA column
// block c), so a row of the strip is one contiguous 64*VW-byte run per 16
// lanes.  The result register r of block c is C[4g + r][VW*i + c].
//
// Few columns (kind 1): each wave owns one row of A and walks it with 16-byte
// loads (neighbouring lanes on neighbouring addresses: "a CUDA matmul"
// section 04), multiplying by the N <= NB columns of B (small, cache
// resident), then reduces its 64 lanes.
//
// Transposed storage.  B stored N x K (a linear layer's weight, C = X W^T):
// in kind 0 a lane's four k values of one column are contiguous in that
// column's row of B^T, one 16-byte load per column (4 lanes cover 64
// contiguous bytes of a row per chunk); in kind 1 the N <= NB rows of B^T
// are read 16 bytes at a time like A's row.  A stored K x M is served by
// kind 0 only (its <= 16 columns are read four bytes at a time; A is small).
#include <cstdint>

#include "gemm_internal.hpp"

namespace sg {
namespace {

// ---------------------------------------------------------------- kind 0 ----
template <int VW, int W>
struct RowsShape {
    static constexpr int NT = 64 * W;
    static constexpr int STRIP = 16 * VW;
    static constexpr int RED = W * VW * 64 * 4;      // floats of the reduction buffer
    static constexpr int LDS_BYTES = RED * 4;
};

// Rows of B in the few-rows kernel and the row of A in the few-columns kernel
// are streamed exactly once: their 8- and 16-byte loads are non-temporal (measured
// +2-6 % on 16 x 14336 x 4096, 4096 x 1 x 4096 and 1 x 2048 x 8192).  The
// column runs of B^T are not: 4 lanes share each 64-byte run, and the hint
// cost 6 % there.
template <int VW, bool VEC>
__device__ __forceinline__ void load_brow(const Problem &p, int k, int gn, float (&v)[VW]) {
#pragma unroll
    for (int c = 0; c < VW; ++c) v[c] = 0.f;
    if (k >= p.K) return;
    const float *src = p.B + (long long)k * p.ldb + gn;
    if (VEC && gn + VW - 1 < p.N) {
        if constexpr (VW == 4) {
            const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(src));
            v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
            return;
        } else if constexpr (VW == 2) {
            typedef float floatx2 __attribute__((ext_vector_type(2)));
            const floatx2 t = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(src));
            v[0] = t[0]; v[1] = t[1];
            return;
        }
    }
#pragma unroll
    for (int c = 0; c < VW; ++c)
        if (gn + c < p.N) v[c] = src[c];
}

// One round of a wave's loads: U 16-wide k-chunks (chunk indices j, j + W,
// ..., j + (U-1)W), for each 4 B rows of VW values and a 4-value A sliver.
template <int VW, int U>
struct RowsRound {
    float b[U][4][VW];
    floatx4 a[U];
};

// B^T stored N x K: the four k values k0 .. k0+3 of column n (zero past K or N).
template <bool VEC>
__device__ __forceinline__ floatx4 load_bcol(const Problem &p, int k0, int n) {
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
    if (n >= p.N || k0 >= p.K) return t;
    const float *src = p.B + (long long)n * p.ldb + k0;
    if (VEC && k0 + 3 < p.K) return *reinterpret_cast<const floatx4 *>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (k0 + e < p.K) t[e] = src[e];
    return t;
}

// VA: rows of A allow 16-byte loads (untransposed A); VB: rows of B allow
// VW-float loads (16-byte loads of B^T's rows with TB).  `arow` walks A's
// row i in steps of `astep` floats (1, or lda for A stored transposed).
template <int VW, int W, int U, bool VA, bool VB, bool TB>
__device__ __forceinline__ void rows_load(const Problem &p, int j, int g, int gn, bool row_ok,
                                          const float *arow, long long astep,
                                          RowsRound<VW, U> &r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k0 = (j + u * W) * 16 + 4 * g;
        if constexpr (TB) {
#pragma unroll
            for (int c = 0; c < VW; ++c) {
                const floatx4 t = load_bcol<VB>(p, k0, gn + c);
#pragma unroll
                for (int s = 0; s < 4; ++s) r.b[u][s][c] = t[s];
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) load_brow<VW, VB>(p, k0 + s, gn, r.b[u][s]);
        }
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
        if (row_ok) {
            if (VA && astep == 1 && k0 + 3 < p.K) {
                a = *reinterpret_cast<const floatx4 *>(arow + k0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (k0 + e < p.K) a[e] = arow[(long long)(k0 + e) * astep];
            }
        }
        r.a[u] = a;
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// IN = 1 / 2: 16-bit inputs in word form (see the 16-bit family): a lane's
// four k-words of A and of column c are the 8 k values of one
// v_mfma_f32_16x16x32 (bfloat16 / float16).
template <int VW, int U, int IN = 0>
__device__ __forceinline__ void rows_mfma(const RowsRound<VW, U> &r, floatx4 (&acc)[VW]) {
    if constexpr (IN != 0) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int c = 0; c < VW; ++c) {
                const floatx4 b = {r.b[u][0][c], r.b[u][1][c], r.b[u][2][c], r.b[u][3][c]};
                if constexpr (IN == 1)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, r.a[u]), __builtin_bit_cast(bf16x8, b), acc[c],
                        0, 0, 0);
                else
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(f16x8, r.a[u]), __builtin_bit_cast(f16x8, b), acc[c],
                        0, 0, 0);
            }
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < VW; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.a[u][s], r.b[u][s][c], acc[c], 0, 0,
                                                              0);
}

// The strip's B columns are streamed once.  Each wave walks its chunks in
// rounds of U with two register sets: the loads of round r + 1 are issued
// before the MFMAs of round r, so a round's memory latency overlaps the
// previous round's arithmetic (loads past K read as zero, so the extra round
// at the end touches no memory).
//
// SPLIT: workgroup (strip, 0, z) runs its strip over rows [z*kslice,
// (z+1)*kslice) of K only, as a product of its own (A and B advanced to the
// slice, K its length), and stores to C + z*stride_c (the split launcher
// points C at a workspace of partial results).
template <int VW, int W, int U, bool VA, bool VB, bool TB, int IN = 0, bool SPLIT = false>
__global__ void __launch_bounds__(64 * W, 1) rows_kernel(Problem p, int strips, int kslice) {
    static_assert(IN == 0 || TB, "16-bit inputs: B transposed (word form)");
    using S = RowsShape<VW, W>;
    __shared__ __attribute__((aligned(16))) float red[S::RED];
    select_batch(p);
    if constexpr (SPLIT) {
        const long long k0 = (long long)blockIdx.z * kslice;
        p.A += p.trans_a ? k0 * p.lda : k0;
        p.B += p.trans_b ? k0 : k0 * p.ldb;
        p.K = (int)((long long)kslice < p.K - k0 ? (long long)kslice : p.K - k0);
        p.C += (long long)blockIdx.z * p.stride_c;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = lane & 15, g = lane >> 4;
    // neighbouring strips share cache lines of B: keep them on one XCD's L2
    const int n0 = xcd_remap(blockIdx.x, strips) * S::STRIP;
    const int gn = n0 + VW * i;
    const bool row_ok = i < p.M;
    // row i of op(A): contiguous, or column i of A stored K x M
    const long long astep = p.trans_a ? p.lda : 1;
    const float *arow = p.A + (row_ok ? (p.trans_a ? (long long)i : (long long)i * p.lda) : 0);

    floatx4 acc[VW];
#pragma unroll
    for (int c = 0; c < VW; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int chunks = (p.K + 15) / 16;
    RowsRound<VW, U> r0, r1;
    rows_load<VW, W, U, VA, VB, TB>(p, wave, g, gn, row_ok, arow, astep, r0);
    for (int j = wave; j < chunks; j += 2 * U * W) {
        rows_load<VW, W, U, VA, VB, TB>(p, j + U * W, g, gn, row_ok, arow, astep, r1);
        pipeline_fence();
        rows_mfma<VW, U, IN>(r0, acc);
        if (j + U * W >= chunks) break;
        rows_load<VW, W, U, VA, VB, TB>(p, j + 2 * U * W, g, gn, row_ok, arow, astep, r0);
        pipeline_fence();
        rows_mfma<VW, U, IN>(r1, acc);
    }

    // fixed-order reduction over the W waves
#pragma unroll
    for (int c = 0; c < VW; ++c)
        *reinterpret_cast<floatx4 *>(red + ((wave * VW + c) * 64 + lane) * 4) = acc[c];
    __syncthreads();
    const bool read_c = (p.beta != 0.f);
    const bool epi = p.has_epilogue();   // bias / activation applied here
    for (int e = tid; e < VW * 64 * 4; e += S::NT) {
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) sum += red[w * VW * 64 * 4 + e];
        const int r = e & 3, l = (e >> 2) & 63, c = e >> 8;
        const int row = 4 * (l >> 4) + r;
        const int col = n0 + VW * (l & 15) + c;
        if (row < p.M && col < p.N) {
            float *dst = p.C + (long long)row * p.ldc + col;
            float out = p.alpha * sum;
            if (read_c) out = fmaf(p.beta, *dst, out);
            if (epi) out = activate(p.act, p.bias ? out + p.bias[col] : out);
            *dst = out;
        }
    }
}

// Split-K of a few-rows product: the sum over the slices in slice order, then
// C = act(alpha * sum + beta * C + bias) as the unsplit kernel's epilogue.
__global__ void __launch_bounds__(256) rows_split_reduce(Problem p, const float *ws, int splits) {
    const long long mn = (long long)p.M * p.N;
    for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < mn;
         e += (long long)gridDim.x * blockDim.x) {
        // slice order kept; loads eight slices ahead of the adds
        float sum = 0.f;
        int z = 0;
        for (; z + 8 <= splits; z += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ws[(z + u) * mn + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; z < splits; ++z) sum += ws[z * mn + e];
        const int row = (int)(e / p.N), col = (int)(e % p.N);
        float *dst = p.C + (long long)row * p.ldc + col;
        float out = p.alpha * sum;
        if (p.beta != 0.f) out = fmaf(p.beta, *dst, out);
        if (p.has_epilogue()) out = activate(p.act, p.bias ? out + p.bias[col] : out);
        *dst = out;
    }
}

// Slices for a split-K launch of a few-rows product, or 1: single products
// whose strips fill under 192 CUs, cut into about 512 workgroups with at
// least two rounds of U chunks per wave in every slice.  kslice: rows of K
// per slice (a multiple of 16, so 16-byte alignment carries over).
template <int VW, int W, int U>
int rows_splits(const Problem &p, int &kslice) {
    kslice = p.K;
    if (p.batch != 1 || p.K == 0) return 1;
    const long long strips = (p.N + 16 * VW - 1) / (16 * VW);
    if (strips >= 192) return 1;
    const long long chunks = (p.K + 15) / 16;
    long long s = (512 + strips - 1) / strips;
    const long long most = chunks / (2LL * W * U);
    if (s > most) s = most;
    if (s < 2) return 1;
    const long long per = (chunks + s - 1) / s;
    kslice = (int)(per * 16);
    return (int)((p.K + kslice - 1) / kslice);
}

template <int VW, int W, int U, bool VA, bool VB, bool TB, int IN = 0, bool SPLIT = false>
hipError_t launch_rows_as(const Problem &p, hipStream_t stream) {
    const int strips = (p.N + 16 * VW - 1) / (16 * VW);
    int kslice = p.K;
    const int splits = SPLIT ? rows_splits<VW, W, U>(p, kslice) : 1;
    if (splits == 1) {
        hipLaunchKernelGGL((rows_kernel<VW, W, U, VA, VB, TB, IN>), dim3(strips, p.batch),
                           dim3(64 * W), 0, stream, p, strips, kslice);
        return hipGetLastError();
    }
    // partial results of the slices: splits x M x N floats
    const long long mn = (long long)p.M * p.N;
    Workspace w;
    hipError_t e = workspace_acquire((size_t)splits * mn * 4, stream, w);
    if (e != hipSuccess) return e;
    float *ws = static_cast<float *>(w.ptr);
    Problem q = p;
    q.C = ws;
    q.ldc = p.N;
    q.stride_c = mn;
    q.alpha = 1.f;
    q.beta = 0.f;
    q.bias = nullptr;
    q.act = SGEMM_ACT_NONE;
    hipLaunchKernelGGL((rows_kernel<VW, W, U, VA, VB, TB, IN, true>), dim3(strips, 1, splits),
                       dim3(64 * W), 0, stream, q, strips, kslice);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const long long blocks = (mn + 255) / 256 < 1024 ? (mn + 255) / 256 : 1024;
        hipLaunchKernelGGL(rows_split_reduce, dim3((unsigned)blocks), dim3(256), 0, stream, p,
                           static_cast<const float *>(ws), splits);
        e = hipGetLastError();
    }
    const hipError_t f = workspace_release(w, stream);
    return e != hipSuccess ? e : f;
}

// 16-bit inputs, few rows: pw is the word-form problem (A untransposed, B
// transposed, K / lda / ldb in 32-bit words); 16-column strips (measured
// faster than 64-column ones for 16-bit inputs at 1 x 14336 x 4096 and
// 16 x 14336 x 4096).
template <int IN>
hipError_t launch_rows16_as(const Problem &pw, hipStream_t stream) {
    const bool va = rows_aligned(pw.A, pw.lda, pw.stride_a, pw.batch, 4);
    const bool vb = rows_aligned(pw.B, pw.ldb, pw.stride_b, pw.batch, 4);
    if (va && vb) return launch_rows_as<1, 16, 4, true, true, true, IN>(pw, stream);
    return launch_rows_as<1, 16, 4, false, false, true, IN>(pw, stream);
}

template <int VW, int W, int U, bool TB, bool SPLIT>
hipError_t launch_rows_tb(const Problem &p, bool va, bool vb, hipStream_t stream) {
    if (va && vb) return launch_rows_as<VW, W, U, true, true, TB, 0, SPLIT>(p, stream);
    if (va) return launch_rows_as<VW, W, U, true, false, TB, 0, SPLIT>(p, stream);
    if (vb) return launch_rows_as<VW, W, U, false, true, TB, 0, SPLIT>(p, stream);
    return launch_rows_as<VW, W, U, false, false, TB, 0, SPLIT>(p, stream);
}

// VEC: wide loads wherever an operand's rows allow them (decided per operand);
// otherwise 4-byte loads throughout.
template <int VW, int W, int U, bool VEC, bool SPLIT = false>
hipError_t launch_rows(const Problem &p, int, hipStream_t stream) {
    const bool va = VEC && !p.trans_a && rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4);
    if (p.trans_b) {
        const bool vb = VEC && rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4);
        return launch_rows_tb<VW, W, U, true, SPLIT>(p, va, vb, stream);
    }
    const bool vb = VEC && rows_aligned(p.B, p.ldb, p.stride_b, p.batch, VW);
    return launch_rows_tb<VW, W, U, false, SPLIT>(p, va, vb, stream);
}

// ---------------------------------------------------------------- kind 1 ----
// One round of a lane's loads: U 4-float chunks of its row of A (k = 4*lane +
// 256u + 0..3) and the matching 4 x NB values of B.
template <int NB, int U>
struct ColsRound {
    floatx4 a[U];
    float b[U][4][NB];
};

// BM (B's mode): 0 any K x N layout, read four bytes at a time; 1 a tight
// K x NB block (ldb == N == NB), so the 4*NB values of four consecutive k are
// contiguous and are read as NB 16-byte loads; 2 B stored transposed (N x K),
// each of its N rows read 16 bytes at a time like A's row; 3 the same, four
// bytes at a time.  VEC: 16-byte loads of A.
template <int NB, int U, bool VEC, int BM>
__device__ __forceinline__ void cols_load(const Problem &p, const float *arow, int kbase,
                                          ColsRound<NB, U> &r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = kbase + 256 * u;
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
        if (VEC && k + 3 < p.K) {
            a = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(arow + k));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (k + e < p.K) a[e] = arow[k + e];
        }
        r.a[u] = a;
        if constexpr (BM >= 2) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                floatx4 t = {0.f, 0.f, 0.f, 0.f};
                if (j < p.N) {
                    const float *src = p.B + (long long)j * p.ldb + k;
                    if (BM == 2 && k + 3 < p.K) {
                        t = *reinterpret_cast<const floatx4 *>(src);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (k + e < p.K) t[e] = src[e];
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) r.b[u][e][j] = t[e];
            }
        } else if (BM == 1 && k + 3 < p.K) {
            const floatx4 *src = reinterpret_cast<const floatx4 *>(p.B + (long long)k * NB);
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const floatx4 v = src[q];
#pragma unroll
                for (int x = 0; x < 4; ++x) r.b[u][(4 * q + x) / NB][(4 * q + x) % NB] = v[x];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float *brow = p.B + (long long)(k + e) * p.ldb;
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    r.b[u][e][j] = (k + e < p.K && j < p.N) ? brow[j] : 0.f;
            }
        }
    }
}

template <int NB, int U>
__device__ __forceinline__ void cols_fma(const ColsRound<NB, U> &r, float (&acc)[NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[j] = fmaf(r.a[u][e], r.b[u][e][j], acc[j]);
}

// One wave per row of A; rounds of U chunks double-buffered as in the
// few-rows kernel (loads past K read as zero and touch no memory).
template <int NB, int W, int U, bool VEC, int BM>
__global__ void __launch_bounds__(64 * W) cols_kernel(Problem p) {
    select_batch(p);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * W + wave;
    if (row >= p.M) return;                       // whole wave leaves together; no barrier below
    const float *arow = p.A + (long long)row * p.lda;
    float acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = 0.f;

    ColsRound<NB, U> r0, r1;
    cols_load<NB, U, VEC, BM>(p, arow, 4 * lane, r0);
    // kw: the wave's base column of A for the round in r0 (uniform over lanes)
    for (int kw = 0; kw < p.K; kw += 2 * 256 * U) {
        cols_load<NB, U, VEC, BM>(p, arow, 4 * lane + kw + 256 * U, r1);
        pipeline_fence();
        cols_fma<NB, U>(r0, acc);
        if (kw + 256 * U >= p.K) break;
        cols_load<NB, U, VEC, BM>(p, arow, 4 * lane + kw + 2 * 256 * U, r0);
        pipeline_fence();
        cols_fma<NB, U>(r1, acc);
    }
    // butterfly reduction over the 64 lanes (fixed order)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        float v = acc[j];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        acc[j] = v;
    }
    const bool read_c = (p.beta != 0.f);
    const bool epi = p.has_epilogue();   // bias / activation applied here
    float *crow = p.C + (long long)row * p.ldc;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (lane == j && j < p.N) {
            float out = p.alpha * acc[j];
            if (read_c) out = fmaf(p.beta, crow[j], out);
            if (epi) out = activate(p.act, p.bias ? out + p.bias[j] : out);
            crow[j] = out;
        }
    }
}

template <int NB, int W, int U, bool VA, int BM>
hipError_t launch_cols_as(const Problem &p, hipStream_t stream) {
    const int blocks = (p.M + W - 1) / W;
    hipLaunchKernelGGL((cols_kernel<NB, W, U, VA, BM>), dim3(blocks, p.batch), dim3(64 * W), 0,
                       stream, p);
    return hipGetLastError();
}

template <int NB, int W, int U, int BM>
hipError_t launch_cols_bm(const Problem &p, bool va, hipStream_t stream) {
    return va ? launch_cols_as<NB, W, U, true, BM>(p, stream)
              : launch_cols_as<NB, W, U, false, BM>(p, stream);
}

// VEC: 16-byte loads of A where its rows allow them, and of B where it is one
// tight K x NB block or stored transposed with aligned rows (decided per
// operand); otherwise 4-byte loads.  A stored transposed is not served.
template <int NB, int W, int U, bool VEC>
hipError_t launch_cols(const Problem &p, int, hipStream_t stream) {
    if (p.trans_a) return hipErrorInvalidValue;
    const bool va = VEC && rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4);
    const bool vb = VEC && rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4);
    if (p.trans_b)
        return vb ? launch_cols_bm<NB, W, U, 2>(p, va, stream)
                  : launch_cols_bm<NB, W, U, 3>(p, va, stream);
    if (vb && p.N == NB && p.ldb == NB) return launch_cols_bm<NB, W, U, 1>(p, va, stream);
    return launch_cols_bm<NB, W, U, 0>(p, va, stream);
}

template <int VW, int W, int U, bool SPLIT = false>
constexpr TileEntry rows_entry() {
    using S = RowsShape<VW, W>;
    // the launchers apply a problem's bias / activation themselves, so the
    // 16-byte launcher is also the fused one
    return TileEntry{{16, 16 * VW, 16 * W, 16, 16 * VW, 0, 0, S::NT, S::LDS_BYTES, 0, 0},
                     &launch_rows<VW, W, U, true, SPLIT>, &launch_rows<VW, W, U, false, SPLIT>, 0,
                     &launch_rows<VW, W, U, true, SPLIT>};
}

template <int NB, int W, int U>
constexpr TileEntry cols_entry() {
    return TileEntry{{W, NB, 256 * U, 1, NB, 1, 0, 64 * W, 0, 0, 0},
                     &launch_cols<NB, W, U, true>, &launch_cols<NB, W, U, false>, 0,
                     &launch_cols<NB, W, U, true>};
}


}  // namespace

hipError_t launch_skinny16(int dtype, const Problem &pw, hipStream_t stream) {
    if (pw.M > 16 || pw.trans_a || !pw.trans_b) return hipErrorInvalidValue;
    return dtype == SGEMM_DTYPE_BF16 ? launch_rows16_as<1>(pw, stream)
                                     : launch_rows16_as<2>(pw, stream);
}

const TileEntry *skinny_tiles(int *count) {
    static const TileEntry tiles[] = {
        rows_entry<1, 16, 4>(),   // 0: 16-column strips
        rows_entry<2, 16, 2>(),   // 1: 32-column strips
        rows_entry<4, 16, 1>(),   // 2: 64-column strips
        rows_entry<2, 8, 4>(),    // 3: 32-column strips, 8 waves
        cols_entry<1, 4, 4>(),    // 4
        cols_entry<2, 4, 4>(),    // 5
        cols_entry<4, 4, 4>(),    // 6
        cols_entry<8, 4, 2>(),    // 7
        cols_entry<16, 4, 2>(),   // 8
        rows_entry<4, 4, 4, true>(),    // 9: 64-column strips, split-K when strips are few
        rows_entry<4, 8, 2, true>(),    // 10: the same, 8 waves
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

// The kind is recorded in the tile descriptor's tm field.
int skinny_kind(int tile) {
    int count = 0;
    const TileEntry *tiles = skinny_tiles(&count);
    return (tile >= 0 && tile < count) ? tiles[tile].desc.tm : -1;
}

// Kind 0 serves every transposition; kind 1 does not read A stored transposed.
bool skinny_fits(int tile, const Problem &p) {
    int count = 0;
    const TileEntry *tiles = skinny_tiles(&count);
    if (tile < 0 || tile >= count) return false;
    return skinny_kind(tile) == 0 ? p.M <= 16 : (p.N <= tiles[tile].desc.bn && !p.trans_a);
}

// Few-rows tile choice, from graph-replay and eager timings over M = 1..16,
// N = 256..14336, K = 1024..16384 with operands larger than the Infinity
// Cache: 64-column strips once they give most CUs a workgroup; 16-column
// strips for B stored transposed (4 lanes read 64 contiguous bytes of a
// column's K run), 32-column strips otherwise; split-K (tile 10) where those
// leave most CUs idle for a long K.
int skinny_pick(const Problem &p) {
    const int M = p.M, N = p.N, K = p.K;
    if (M <= 16) {
        if ((N + 63) / 64 >= 160) return 2;
        const bool split_ok = p.batch == 1;
        if (p.trans_b) {
            if (split_ok && K >= 8192 && N <= 2048) return 10;
            return N >= 8192 ? 1 : 0;
        }
        if (split_ok && ((K >= 4096 && N <= 2048) || (K >= 8192 && N <= 4096))) return 10;
        return 1;
    }
    if (N <= 16 && !p.trans_a) {
        int count = 0;
        const TileEntry *tiles = skinny_tiles(&count);
        for (int t = 0; t < count; ++t)
            if (skinny_kind(t) == 1 && N <= tiles[t].desc.bn) return t;
    }
    return -1;
}

}  // namespace sg
