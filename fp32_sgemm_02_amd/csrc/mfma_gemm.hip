// mfma_gemm.hip -- fp32 SGEMM on the CDNA4 matrix cores (v_mfma_f32_16x16x4_f32).
//
// C = alpha * (A * B) + beta * C, row-major fp32 with leading dimensions.
//
// The method is the tiling hierarchy the pages build up, mapped onto gfx950:
//   * every cell of C is an independent dot product, so workgroups own
//     disjoint BM x BN tiles of C ("a CUDA matmul" section 01: blocks tile the
//     output; "The GEMM Scrapbook" introduction: the cells are independent);
//   * A and B are staged through on-chip memory one K-slice at a time and
//     reused from there ("a CUDA matmul" section 05; Scrapbook shared-memory
//     chapter), here in LDS, with two buffers so the next slice is fetched
//     while the current one is consumed (Scrapbook warptiling chapter, double
//     buffering);
//   * global loads are 16-byte vectors over contiguous addresses of
//     neighbouring lanes (coalescing: "a CUDA matmul" section 04, "The 1%
//     kernel" section 5; 128-bit loads: Scrapbook vectorisation chapter);
//   * each wave owns an explicit WM x WN sub-tile (Scrapbook warptiling
//     chapter), which it computes as a sum of outer products over k
//     (Scrapbook 2D-tiling chapter) -- here each 16 x 16 x 4 block of that sum
//     is one MFMA instruction instead of 1024 scalar FMAs;
//   * LDS rows of A are padded so that the 16-byte fragment reads of a wave
//     hit distinct banks (Scrapbook warptiling chapter, bank conflicts).
//
// Lane layout of v_mfma_f32_16x16x4_f32 (wave64, lane l, i = l % 16, g = l / 16):
//   A operand: A[i][g], B operand: B[g][i], result register r: D[4g + r][i].
// Two re-labellings make every LDS access a 16-byte read:
//   * k: in MFMA step s of a 16-wide k-chunk, lane group g supplies
//     k = 4g + s, so a lane's A values for the four steps are 4 consecutive
//     floats of one A row;
//   * n: the four MFMA column blocks c = 0..3 of a 64-column group take
//     columns 4i + c, so a lane's B values for the four blocks are 4
//     consecutive floats of one B row, and its results for one row of C are 4
//     consecutive columns (one 16-byte store).
// Both only permute the terms of each dot product and the columns of C, so
// every cell still receives exactly the K products A[m][k]*B[k][n].
#include "gemm_internal.hpp"

namespace sg {
namespace {

template <int BM, int BN, int BK, int WM, int WN>
struct MfmaShape {
    static constexpr int WAVES_M = BM / WM;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int RB = WM / 16;          // 16-row MFMA blocks per wave
    static constexpr int CG = WN / 64;          // 64-column groups per wave
    static constexpr int AS = BK + 4;           // LDS row stride of the A tile (floats)
    static constexpr int BS = BN + 4;           // LDS row stride of the B tile (floats)
    static constexpr int A_STAGE = BM * AS;
    static constexpr int B_STAGE = BK * BS;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int A_VEC = BM * BK / 4 / NT;   // 16-byte loads per thread per stage
    static constexpr int B_VEC = BK * BN / 4 / NT;
    static_assert(BM % WM == 0 && BN % WN == 0, "wave grid must tile the block");
    static_assert(WM % 16 == 0 && WN % 64 == 0, "wave tile: 16-row x 64-column units");
    static_assert(BK % 16 == 0, "K step is a multiple of 16");
    static_assert(A_VEC * NT * 4 == BM * BK && B_VEC * NT * 4 == BK * BN,
                  "tile loads must divide evenly over the workgroup");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
};

// Load one 4-float chunk of A starting at (row gm, column gk).  GUARD: zero
// outside [0,M) x [0,K).  VEC: one 16-byte load when the chunk is whole.
template <bool GUARD, bool VEC>
__device__ __forceinline__ floatx4 load_a(const Problem &p, int gm, int gk) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (GUARD && gm >= p.M) return v;
    const float *src = p.A + (long long)gm * p.lda + gk;
    if (VEC && (!GUARD || gk + 3 < p.K)) return *reinterpret_cast<const floatx4 *>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (!GUARD || gk + e < p.K) v[e] = src[e];
    return v;
}

// Load one 4-float chunk of B starting at (row gk, column gn).
template <bool GUARD, bool VEC>
__device__ __forceinline__ floatx4 load_b(const Problem &p, int gk, int gn) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (GUARD && gk >= p.K) return v;
    const float *src = p.B + (long long)gk * p.ldb + gn;
    if (VEC && (!GUARD || gn + 3 < p.N)) return *reinterpret_cast<const floatx4 *>(src);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (!GUARD || gn + e < p.N) v[e] = src[e];
    return v;
}

template <int BM, int BN, int BK, int WM, int WN, bool GUARD, bool VEC>
__device__ __forceinline__ void global_to_regs(const Problem &p, int m0, int n0, int k0,
                                               int tid, floatx4 (&ra)[MfmaShape<BM, BN, BK, WM, WN>::A_VEC],
                                               floatx4 (&rb)[MfmaShape<BM, BN, BK, WM, WN>::B_VEC]) {
    using S = MfmaShape<BM, BN, BK, WM, WN>;
#pragma unroll
    for (int v = 0; v < S::A_VEC; ++v) {
        const int c = tid + v * S::NT;
        const int row = c / (BK / 4), kq = c % (BK / 4);
        ra[v] = load_a<GUARD, VEC>(p, m0 + row, k0 + 4 * kq);
    }
#pragma unroll
    for (int v = 0; v < S::B_VEC; ++v) {
        const int c = tid + v * S::NT;
        const int krow = c / (BN / 4), nq = c % (BN / 4);
        rb[v] = load_b<GUARD, VEC>(p, k0 + krow, n0 + 4 * nq);
    }
}

template <int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void regs_to_lds(float *stage, int tid,
                                            const floatx4 (&ra)[MfmaShape<BM, BN, BK, WM, WN>::A_VEC],
                                            const floatx4 (&rb)[MfmaShape<BM, BN, BK, WM, WN>::B_VEC]) {
    using S = MfmaShape<BM, BN, BK, WM, WN>;
    float *As = stage;
    float *Bs = stage + S::A_STAGE;
#pragma unroll
    for (int v = 0; v < S::A_VEC; ++v) {
        const int c = tid + v * S::NT;
        const int row = c / (BK / 4), kq = c % (BK / 4);
        *reinterpret_cast<floatx4 *>(As + row * S::AS + 4 * kq) = ra[v];
    }
#pragma unroll
    for (int v = 0; v < S::B_VEC; ++v) {
        const int c = tid + v * S::NT;
        const int krow = c / (BN / 4), nq = c % (BN / 4);
        *reinterpret_cast<floatx4 *>(Bs + krow * S::BS + 4 * nq) = rb[v];
    }
}

// One BK-deep stage of the wave's outer-product accumulation.
template <int BM, int BN, int BK, int WM, int WN>
__device__ __forceinline__ void mfma_stage(const float *stage, int lane, int wr, int wc,
                                           floatx4 (&acc)[WM / 16][WN / 16]) {
    using S = MfmaShape<BM, BN, BK, WM, WN>;
    const float *As = stage + (wr * WM + (lane & 15)) * S::AS + 4 * (lane >> 4);
    const float *Bs = stage + S::A_STAGE + 4 * (lane >> 4) * S::BS + wc * WN + 4 * (lane & 15);
#pragma unroll
    for (int kc = 0; kc < BK / 16; ++kc) {
        floatx4 a[S::RB];
#pragma unroll
        for (int rb = 0; rb < S::RB; ++rb)
            a[rb] = *reinterpret_cast<const floatx4 *>(As + rb * 16 * S::AS + kc * 16);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            floatx4 b[S::CG];
#pragma unroll
            for (int cg = 0; cg < S::CG; ++cg)
                b[cg] = *reinterpret_cast<const floatx4 *>(Bs + (kc * 16 + s) * S::BS + cg * 64);
#pragma unroll
            for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
                for (int cg = 0; cg < S::CG; ++cg)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[rb][cg * 4 + c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            a[rb][s], b[cg][c], acc[rb][cg * 4 + c], 0, 0, 0);
        }
    }
}

// alpha/beta epilogue and stores.  beta == 0 never reads C.
template <int WM, int WN, bool GUARD, bool VEC>
__device__ __forceinline__ void store_tile(const Problem &p, int row0, int col0, int lane,
                                           const floatx4 (&acc)[WM / 16][WN / 16]) {
    const int i = lane & 15, g = lane >> 4;
    const bool read_c = (p.beta != 0.f);
#pragma unroll
    for (int rb = 0; rb < WM / 16; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int gm = row0 + rb * 16 + 4 * g + r;
            if (GUARD && gm >= p.M) continue;
            float *crow = p.C + (long long)gm * p.ldc;
#pragma unroll
            for (int cg = 0; cg < WN / 64; ++cg) {
                const int gn = col0 + cg * 64 + 4 * i;
                floatx4 v;
#pragma unroll
                for (int c = 0; c < 4; ++c) v[c] = p.alpha * acc[rb][cg * 4 + c][r];
                if (VEC && (!GUARD || gn + 3 < p.N)) {
                    floatx4 *dst = reinterpret_cast<floatx4 *>(crow + gn);
                    if (read_c) {
                        const floatx4 old = *dst;
#pragma unroll
                        for (int c = 0; c < 4; ++c) v[c] = fmaf(p.beta, old[c], v[c]);
                    }
                    *dst = v;
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (GUARD && gn + c >= p.N) continue;
                        float out = v[c];
                        if (read_c) out = fmaf(p.beta, crow[gn + c], out);
                        crow[gn + c] = out;
                    }
                }
            }
        }
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
__global__ void __launch_bounds__((MfmaShape<BM, BN, BK, WM, WN>::NT), 1)
mfma_sgemm_kernel(Problem p, int tiles_m, int tiles_n, int group_m) {
    using S = MfmaShape<BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) float smem[2 * S::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave / S::WAVES_N, wc = wave % S::WAVES_N;

    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    floatx4 acc[WM / 16][WN / 16];
#pragma unroll
    for (int a = 0; a < WM / 16; ++a)
#pragma unroll
        for (int b = 0; b < WN / 16; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    floatx4 ra[S::A_VEC], rb[S::B_VEC];
    const int nk = (p.K + BK - 1) / BK;

    auto fetch = [&](int t) {
        const int k0 = t * BK;
        if (interior && k0 + BK <= p.K)
            global_to_regs<BM, BN, BK, WM, WN, false, VEC>(p, m0, n0, k0, tid, ra, rb);
        else
            global_to_regs<BM, BN, BK, WM, WN, true, VEC>(p, m0, n0, k0, tid, ra, rb);
    };

    fetch(0);
    regs_to_lds<BM, BN, BK, WM, WN>(smem, tid, ra, rb);
    __syncthreads();

    for (int t = 0; t < nk; ++t) {
        const bool more = (t + 1 < nk);
        if (more) fetch(t + 1);
        mfma_stage<BM, BN, BK, WM, WN>(smem + (t & 1) * S::STAGE, lane, wr, wc, acc);
        if (more) regs_to_lds<BM, BN, BK, WM, WN>(smem + ((t + 1) & 1) * S::STAGE, tid, ra, rb);
        // one barrier per stage: it publishes stage t+1 and, because the next
        // iteration writes the buffer just read, also retires stage t.
        __syncthreads();
    }

    const int row0 = m0 + wr * WM, col0 = n0 + wc * WN;
    if (interior)
        store_tile<WM, WN, false, VEC>(p, row0, col0, lane, acc);
    else
        store_tile<WM, WN, true, VEC>(p, row0, col0, lane, acc);
}

template <int BM, int BN, int BK, int WM, int WN, bool VEC>
hipError_t launch_mfma(const Problem &p, int group_m, hipStream_t stream) {
    using S = MfmaShape<BM, BN, BK, WM, WN>;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    const long long tiles = (long long)tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (group_m <= 0) group_m = 4;
    hipLaunchKernelGGL((mfma_sgemm_kernel<BM, BN, BK, WM, WN, VEC>), dim3((unsigned)tiles),
                       dim3(S::NT), 0, stream, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN>
constexpr TileEntry mfma_entry() {
    using S = MfmaShape<BM, BN, BK, WM, WN>;
    return TileEntry{{BM, BN, BK, WM, WN, 0, 0, S::NT, S::LDS_BYTES},
                     &launch_mfma<BM, BN, BK, WM, WN, true>,
                     &launch_mfma<BM, BN, BK, WM, WN, false>};
}

}  // namespace

// Compiled tile configurations (index = sgemm_config.tile for the MFMA family).
const TileEntry *mfma_tiles(int *count) {
    static const TileEntry tiles[] = {
        mfma_entry<256, 256, 32, 128, 128>(),   // 0: 4 waves, 256 accumulators per lane
        mfma_entry<256, 256, 16, 128, 128>(),   // 1
        mfma_entry<256, 128, 16, 128, 64>(),    // 2: 4 waves, 128 accumulators per lane
        mfma_entry<128, 128, 32, 64, 64>(),     // 3
        mfma_entry<128, 128, 16, 64, 64>(),     // 4
        mfma_entry<256, 256, 32, 128, 64>(),    // 5: 8 waves
        mfma_entry<128, 256, 32, 64, 128>(),    // 6
        mfma_entry<64, 64, 32, 32, 64>(),       // 7: small problems
        mfma_entry<128, 64, 32, 64, 64>(),      // 8
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
