// mfma_gemm16.hip -- GEMM with 16-bit inputs (bfloat16 or float16 A and B),
// fp32 accumulation and fp32 C: C = alpha * op(A) * op(B) + beta * C.
//
// The reduced-precision matrix instructions the fine print of "The GEMM
// Scrapbook" points to (tensor cores; here v_mfma_f32_16x16x32_{bf16,f16}),
// with the same tiling hierarchy as the fp32 path.
//
// Two kinds of kernel:
//   * the direct-load MFMA tiles of direct_kernel.hpp with IN = 1 / 2, for A
//     untransposed and B transposed (N x K; the weight layout of a linear
//     layer, C = X W^T) with K, lda, ldb even and A, B 4-byte aligned: both
//     operands are then matrices of 32-bit words along k;
//   * a generic tiled kernel for every other layout and alignment, which
//     decodes the 16-bit values to fp32 on their way into LDS and runs 4 x 4
//     fp32 FMA micro-tiles per thread (correct for any shape; not tuned).
#include "direct_kernel.hpp"

namespace sg {
namespace {

// ---- direct-load tiles ---------------------------------------------------------
// TILE16(BM, BN, BK_WORDS, WM, WN, NBUF, KG, EFF): the fp32 kernel's tile
// with BK counted in words (2 k values each).  EFF: % of the 16-bit peak
// measured on whole-GPU shapes (4096^3 and the MLP shapes; dispatch cost
// model).
#define TILES16(X)                              \
    X(256, 256, 32, 128, 64, 2, 1, 48)          \
    X(256, 256, 16, 128, 64, 2, 1, 44)          \
    X(256, 128, 32, 64, 64, 2, 1, 41)           \
    X(128, 128, 32, 32, 64, 2, 1, 41)           \
    X(128, 128, 32, 64, 64, 2, 2, 38)           \
    X(64, 64, 32, 32, 64, 2, 2, 35)            \
    X(256, 256, 32, 64, 128, 2, 1, 50)

struct Tile16 {
    sgemm_tile_desc desc;
    LaunchFn bf16, f16;
    int eff_pct;
};

#define TILE16_ENTRY(BM, BN, BK, WM, WN, NBUF, KG, EFF)                                        \
    Tile16{{BM, BN, 2 * BK, WM, WN, 0, 0,                                                      \
            DirectShape<BM, BN, BK, WM, WN, NBUF, 4, 4, KG, true, false, false, 1>::NT,          \
            DirectShape<BM, BN, BK, WM, WN, NBUF, 4, 4, KG, true, false, false, 1>::LDS_BYTES,   \
            NBUF, SGEMM_TILE_DIRECT | SGEMM_TILE_TRANS_B},                                      \
           &launch_direct16<BM, BN, BK, WM, WN, NBUF, KG, 1>,                                   \
           &launch_direct16<BM, BN, BK, WM, WN, NBUF, KG, 2>, EFF},

const Tile16 kTiles16[] = {TILES16(TILE16_ENTRY)};
constexpr int kTiles16Count = sizeof(kTiles16) / sizeof(kTiles16[0]);

// ---- generic kernel -----------------------------------------------------------
// The value of a 16-bit float (IN 1: bfloat16, the high half of a binary32;
// IN 2: IEEE binary16).
template <int IN>
__device__ __forceinline__ float decode16(unsigned short h) {
    if constexpr (IN == 1)
        return __uint_as_float((unsigned)h << 16);
    else
        return (float)__builtin_bit_cast(_Float16, h);
}

constexpr int G_BM = 64, G_BN = 64, G_BK = 16;

// 256 threads, a 64 x 64 tile of C, thread (ty, tx) owns rows ty + 16r and
// columns tx + 16c (r, c < 4).  op(A) and op(B) are staged k-major in LDS as
// fp32 (As[k][m], Bs[k][n]); loads past M, N or K read as zero.
template <int IN>
__global__ void __launch_bounds__(256) gemm16_generic_kernel(Problem16 p) {
    __shared__ float As[G_BK][G_BM + 1];
    __shared__ float Bs[G_BK][G_BN + 1];
    const long long b = blockIdx.z;
    const unsigned short *A = p.A + b * p.stride_a;
    const unsigned short *B = p.B + b * p.stride_b;
    float *C = p.C + b * p.stride_c;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const int m0 = blockIdx.y * G_BM, n0 = blockIdx.x * G_BN;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += G_BK) {
        for (int e = threadIdx.x; e < G_BK * G_BM; e += 256) {
            const int kk = e / G_BM, mm = e % G_BM;
            const int m = m0 + mm, k = k0 + kk;
            float v = 0.f;
            if (m < p.M && k < p.K)
                v = decode16<IN>(p.trans_a ? A[(long long)k * p.lda + m]
                                           : A[(long long)m * p.lda + k]);
            As[kk][mm] = v;
        }
        for (int e = threadIdx.x; e < G_BK * G_BN; e += 256) {
            const int kk = e / G_BN, nn = e % G_BN;
            const int n = n0 + nn, k = k0 + kk;
            float v = 0.f;
            if (n < p.N && k < p.K)
                v = decode16<IN>(p.trans_b ? B[(long long)n * p.ldb + k]
                                           : B[(long long)k * p.ldb + n]);
            Bs[kk][nn] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < G_BK; ++kk) {
            float a[4], bv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = As[kk][ty + 16 * r];
#pragma unroll
            for (int c = 0; c < 4; ++c) bv[c] = Bs[kk][tx + 16 * c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], bv[c], acc[r][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = m0 + ty + 16 * r;
        if (m >= p.M) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int n = n0 + tx + 16 * c;
            if (n >= p.N) continue;
            float *dst = C + (long long)m * p.ldc + n;
            float out = p.alpha * acc[r][c];
            if (p.beta != 0.f) out = fmaf(p.beta, *dst, out);
            *dst = out;
        }
    }
}

}  // namespace

int tiles16_count() { return kTiles16Count; }

const sgemm_tile_desc *tile16_desc(int tile) {
    return (tile >= 0 && tile < kTiles16Count) ? &kTiles16[tile].desc : nullptr;
}

int tile16_eff(int tile) { return kTiles16[tile].eff_pct; }

hipError_t launch_tile16(int tile, int dtype, const Problem &pw, int group_m,
                         hipStream_t stream) {
    if (tile < 0 || tile >= kTiles16Count) return hipErrorInvalidValue;
    const Tile16 &t = kTiles16[tile];
    return (dtype == SGEMM_DTYPE_BF16 ? t.bf16 : t.f16)(pw, group_m, stream);
}

hipError_t launch_generic16(int dtype, const Problem16 &p, hipStream_t stream) {
    const unsigned gx = (unsigned)((p.N + G_BN - 1) / G_BN);
    const unsigned gy = (unsigned)((p.M + G_BM - 1) / G_BM);
    if (gy > 65535u) return hipErrorInvalidConfiguration;
    for (int b0 = 0; b0 < p.batch; b0 += kMaxBatchPerLaunch) {
        Problem16 q = p;
        q.batch = p.batch - b0 < kMaxBatchPerLaunch ? p.batch - b0 : kMaxBatchPerLaunch;
        q.A += b0 * p.stride_a;
        q.B += b0 * p.stride_b;
        q.C += b0 * p.stride_c;
        if (dtype == SGEMM_DTYPE_BF16)
            hipLaunchKernelGGL(gemm16_generic_kernel<1>, dim3(gx, gy, q.batch), dim3(256), 0,
                               stream, q);
        else
            hipLaunchKernelGGL(gemm16_generic_kernel<2>, dim3(gx, gy, q.batch), dim3(256), 0,
                               stream, q);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sg
