// valu_gemm.hip -- fp32 SGEMM on the vector ALUs: per-lane register
// micro-tiles of plain fp32 FMAs.  This is the comparison family for the
// matrix-core kernels; both compute the same products in fp32.
//
// Design, following the pages' register-blocking ladder and mapped to wave64:
//   * each lane owns a TM x TN = 8 x 8 patch of C held in 64 accumulators and,
//     per k, loads a sliver of 8 values of A and 8 of B and forms their outer
//     product with 64 FMAs ("The GEMM Scrapbook", 2D-tiling chapter: matmul
//     as a sum of outer products);
//   * the A tile is stored transposed (k-major) in LDS while it is written, so
//     that a lane's 8-value sliver of A is two 16-byte LDS reads (Scrapbook
//     vectorisation chapter);
//   * a wave of 64 lanes owns a 64 x 64 wave tile (8 x 8 lanes), the explicit
//     middle level of the hierarchy (Scrapbook warptiling chapter); a lane's 8
//     rows are two runs of 4 split 32 apart (likewise its 8 columns), so the 8
//     lanes that read LDS together cover 128 contiguous bytes and hit distinct
//     banks;
//   * two LDS buffers: the next K-slice is fetched from global memory while
//     the current one is consumed and written to the other buffer half-way
//     through the slice (Scrapbook warptiling chapter, double buffering), one
//     barrier per slice; the next k's slivers are read from LDS while the
//     current k's 64 FMAs run.
// The code is built with packed fp32 instructions disabled, so each FMA is a
// plain v_fma_f32; the family's ceiling is half the chip's packed fp32 rate.
#include "gemm_internal.hpp"

namespace sg {
namespace {

template <int BM, int BN, int BK>
struct ValuShape {
    static constexpr int WAVES_M = BM / 64;
    static constexpr int WAVES_N = BN / 64;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int AS = BM + 4;     // LDS row stride of the k-major A tile
    static constexpr int BS = BN + 4;     // LDS row stride of the B tile
    static constexpr int A_STAGE = BK * AS;
    static constexpr int B_STAGE = BK * BS;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_BYTES = 2 * STAGE * 4;
    static constexpr int A_VEC = BM * BK / 4 / NT;
    static constexpr int B_VEC = BK * BN / 4 / NT;
    static_assert(BM % 64 == 0 && BN % 64 == 0, "64 x 64 wave tiles");
    static_assert(BK == 16, "A loads map 16 rows x 4 chunks per wave");
    static_assert(A_VEC * NT * 4 == BM * BK && B_VEC * NT * 4 == BK * BN, "even load split");
    static_assert(BM % (16 * (NT / 64)) == 0, "A rows split evenly over waves");
};

// Guarded loads read a clamped (always valid) address and select zero outside
// the matrix, so edge tiles do not diverge; only a 16-byte chunk straddling
// K (or N) is read element by element.
template <bool GUARD, bool VEC>
__device__ __forceinline__ floatx4 vload_a(const Problem &p, int gm, int gk) {
    if (!GUARD) {
        const float *src = p.A + (long long)gm * p.lda + gk;
        if (VEC) return *reinterpret_cast<const floatx4 *>(src);
        return floatx4{src[0], src[1], src[2], src[3]};
    }
    const bool row_ok = gm < p.M;
    const float *row = p.A + (row_ok ? (long long)gm * p.lda : 0);
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (VEC) {
        const bool whole = row_ok && gk + 3 < p.K;
        const floatx4 x = *reinterpret_cast<const floatx4 *>(row + (whole ? gk : 0));
        if (whole) v = x;
        else if (row_ok && gk < p.K) {
#pragma unroll
            for (int e = 0; e < 3; ++e)
                if (gk + e < p.K) v[e] = row[gk + e];
        }
        return v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool ok = row_ok && gk + e < p.K;
        const float x = row[ok ? gk + e : 0];
        v[e] = ok ? x : 0.f;
    }
    return v;
}

template <bool GUARD, bool VEC>
__device__ __forceinline__ floatx4 vload_b(const Problem &p, int gk, int gn) {
    if (!GUARD) {
        const float *src = p.B + (long long)gk * p.ldb + gn;
        if (VEC) return *reinterpret_cast<const floatx4 *>(src);
        return floatx4{src[0], src[1], src[2], src[3]};
    }
    const bool row_ok = gk < p.K;
    const float *row = p.B + (row_ok ? (long long)gk * p.ldb : 0);
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (VEC) {
        const bool whole = row_ok && gn + 3 < p.N;
        const floatx4 x = *reinterpret_cast<const floatx4 *>(row + (whole ? gn : 0));
        if (whole) v = x;
        else if (row_ok && gn < p.N) {
#pragma unroll
            for (int e = 0; e < 3; ++e)
                if (gn + e < p.N) v[e] = row[gn + e];
        }
        return v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bool ok = row_ok && gn + e < p.N;
        const float x = row[ok ? gn + e : 0];
        v[e] = ok ? x : 0.f;
    }
    return v;
}

// A chunk v of a thread: wave w covers 16 consecutive rows x 4 k-chunks per
// pass (lane & 15 = row, lane >> 4 = chunk), so that the transposed LDS
// writes of lanes 0..31 land in 32 distinct banks.
template <int BM, int BN, int BK>
__device__ __forceinline__ void a_chunk(int tid, int v, int &row, int &kq) {
    using S = ValuShape<BM, BN, BK>;
    const int lane = tid & 63, wave = tid >> 6;
    row = (v * (S::NT / 64) + wave) * 16 + (lane & 15);
    kq = lane >> 4;
}

template <int BM, int BN, int BK, bool GUARD, bool VEC>
__device__ __forceinline__ void vfetch(const Problem &p, int m0, int n0, int k0, int tid,
                                       floatx4 (&ra)[ValuShape<BM, BN, BK>::A_VEC],
                                       floatx4 (&rb)[ValuShape<BM, BN, BK>::B_VEC]) {
    using S = ValuShape<BM, BN, BK>;
#pragma unroll
    for (int v = 0; v < S::A_VEC; ++v) {
        int row, kq;
        a_chunk<BM, BN, BK>(tid, v, row, kq);
        ra[v] = vload_a<GUARD, VEC>(p, m0 + row, k0 + 4 * kq);
    }
#pragma unroll
    for (int v = 0; v < S::B_VEC; ++v) {
        const int c = tid + v * S::NT;
        const int krow = c / (BN / 4), nq = c % (BN / 4);
        rb[v] = vload_b<GUARD, VEC>(p, k0 + krow, n0 + 4 * nq);
    }
}

template <int BM, int BN, int BK>
__device__ __forceinline__ void vstore_lds(float *stage, int tid,
                                           const floatx4 (&ra)[ValuShape<BM, BN, BK>::A_VEC],
                                           const floatx4 (&rb)[ValuShape<BM, BN, BK>::B_VEC]) {
    using S = ValuShape<BM, BN, BK>;
    float *As = stage;
    float *Bs = stage + S::A_STAGE;
#pragma unroll
    for (int v = 0; v < S::A_VEC; ++v) {
        int row, kq;
        a_chunk<BM, BN, BK>(tid, v, row, kq);
#pragma unroll
        for (int e = 0; e < 4; ++e) As[(4 * kq + e) * S::AS + row] = ra[v][e];
    }
#pragma unroll
    for (int v = 0; v < S::B_VEC; ++v) {
        const int c = tid + v * S::NT;
        const int krow = c / (BN / 4), nq = c % (BN / 4);
        *reinterpret_cast<floatx4 *>(Bs + krow * S::BS + 4 * nq) = rb[v];
    }
}

template <int BM, int BN, int BK, bool VEC>
__global__ void __launch_bounds__((ValuShape<BM, BN, BK>::NT), 2)
valu_sgemm_kernel(Problem p, int tiles_m, int tiles_n, int group_m) {
    using S = ValuShape<BM, BN, BK>;
    __shared__ __attribute__((aligned(16))) float smem[2 * S::STAGE];
    select_batch(p);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / S::WAVES_N, wc = wave % S::WAVES_N;
    const int ty = lane >> 3, tx = lane & 7;

    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    float acc_flat[64];
    float(&acc)[8][8] = *reinterpret_cast<float(*)[8][8]>(acc_flat);
#pragma unroll
    for (int i = 0; i < 64; ++i) acc_flat[i] = 0.f;

    floatx4 ra[S::A_VEC], rb[S::B_VEC];
    const int nk = (p.K + BK - 1) / BK;
    auto fetch = [&](int t) {
        const int k0 = t * BK;
        if (interior && k0 + BK <= p.K)
            vfetch<BM, BN, BK, false, VEC>(p, m0, n0, k0, tid, ra, rb);
        else
            vfetch<BM, BN, BK, true, VEC>(p, m0, n0, k0, tid, ra, rb);
    };

    const int a_off = wr * 64 + 4 * ty;
    const int b_off = wc * 64 + 4 * tx;

    // the lane's slivers for one k: A rows a_off + {0..3}, +32; B columns b_off + {0..3}, +32
    struct Sliver {
        floatx4 a0, a1, b0, b1;
    };
    auto read_sliver = [&](const float *stage, int k, Sliver &v) {
        const float *As = stage + k * S::AS + a_off;
        const float *Bs = stage + S::A_STAGE + k * S::BS + b_off;
        v.a0 = *reinterpret_cast<const floatx4 *>(As);
        v.a1 = *reinterpret_cast<const floatx4 *>(As + 32);
        v.b0 = *reinterpret_cast<const floatx4 *>(Bs);
        v.b1 = *reinterpret_cast<const floatx4 *>(Bs + 32);
    };

    fetch(0);
    vstore_lds<BM, BN, BK>(smem, tid, ra, rb);
    __syncthreads();
    Sliver cur, nxt;
    read_sliver(smem, 0, cur);
    for (int t = 0; t < nk; ++t) {
        const bool more = (t + 1 < nk);
        if (more) fetch(t + 1);
        const float *stage = smem + (t & 1) * S::STAGE;
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            if (k + 1 < BK) read_sliver(stage, k + 1, nxt);
            const float a[8] = {cur.a0[0], cur.a0[1], cur.a0[2], cur.a0[3],
                                cur.a1[0], cur.a1[1], cur.a1[2], cur.a1[3]};
            const float b[8] = {cur.b0[0], cur.b0[1], cur.b0[2], cur.b0[3],
                                cur.b1[0], cur.b1[1], cur.b1[2], cur.b1[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            // the other buffer was last read in stage t - 1, before the
            // barrier that closed it: the next stage can be written now
            if (k == BK / 2 && more)
                vstore_lds<BM, BN, BK>(smem + ((t + 1) & 1) * S::STAGE, tid, ra, rb);
            pipeline_fence(acc_flat);
            if (k + 1 < BK) cur = nxt;
        }
        __syncthreads();
        if (more) read_sliver(smem + ((t + 1) & 1) * S::STAGE, 0, cur);
    }

    // epilogue: alpha/beta; beta == 0 never reads C
    const bool read_c = (p.beta != 0.f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int gm = m0 + a_off + (i & 3) + (i >> 2) * 32;
        if (!interior && gm >= p.M) continue;
        float *crow = p.C + (long long)gm * p.ldc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int gn = n0 + b_off + 32 * h;
            floatx4 v;
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = p.alpha * acc[i][4 * h + c];
            if (VEC && (interior || gn + 3 < p.N)) {
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
                    if (!interior && gn + c >= p.N) continue;
                    float out = v[c];
                    if (read_c) out = fmaf(p.beta, crow[gn + c], out);
                    crow[gn + c] = out;
                }
            }
        }
    }
}

template <int BM, int BN, int BK, bool VEC>
hipError_t launch_valu(const Problem &p, int group_m, hipStream_t stream) {
    using S = ValuShape<BM, BN, BK>;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    const long long tiles = (long long)tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (group_m <= 0) group_m = 8;
    hipLaunchKernelGGL((valu_sgemm_kernel<BM, BN, BK, VEC>), dim3((unsigned)tiles, p.batch),
                       dim3(S::NT),
                       0, stream, p, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

template <int BM, int BN, int BK>
constexpr TileEntry valu_entry() {
    using S = ValuShape<BM, BN, BK>;
    return TileEntry{{BM, BN, BK, 64, 64, 8, 8, S::NT, S::LDS_BYTES, 2, 0},
                     &launch_valu<BM, BN, BK, true>, &launch_valu<BM, BN, BK, false>};
}

}  // namespace

const TileEntry *valu_tiles(int *count) {
    static const TileEntry tiles[] = {
        valu_entry<128, 128, 16>(),   // 0: 4 waves
        valu_entry<64, 64, 16>(),     // 1: 1 wave, small problems
        valu_entry<128, 64, 16>(),    // 2
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
