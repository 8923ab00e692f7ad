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
//     chapter), here in LDS, with two or three buffers so the next slices are
//     fetched while the current one is consumed (Scrapbook warptiling chapter,
//     double buffering);
//   * global loads are 16-byte vectors over contiguous addresses of
//     neighbouring lanes (coalescing: "a CUDA matmul" section 04, "The 1%
//     kernel" section 5; 128-bit loads: Scrapbook vectorisation chapter);
//   * each wave owns an explicit WM x WN sub-tile (Scrapbook warptiling
//     chapter), which it computes as a sum of outer products over k
//     (Scrapbook 2D-tiling chapter) -- here each 16 x 16 x 4 block of that sum
//     is one MFMA instruction instead of 1024 scalar FMAs;
//   * LDS rows of A are padded (B rows are not) so that the 16-byte fragment
//     reads of a wave hit distinct banks (Scrapbook warptiling chapter, bank
//     conflicts); the strides are the ones measured conflict-free on gfx950.
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

// BM x BN workgroup tile, BK-deep K stages, WM x WN wave tiles, NBUF LDS
// stages in a ring, OCC = waves per SIMD the register budget is sized for.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int OCC>
struct MfmaShape {
    static constexpr int WAVES_M = BM / WM;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int RB = WM / 16;          // 16-row MFMA blocks per wave
    static constexpr int CG = WN / 64;          // 64-column groups per wave
    static constexpr int KC = BK / 16;          // 16-wide k-chunks per stage
    // LDS row strides (floats), chosen for conflict-free 16-byte fragment
    // reads on gfx950 (measured with SQ_LDS_BANK_CONFLICT): A rows padded by 8
    // floats (16 rows x 4 chunks read together), B rows unpadded (the four
    // row groups of a B read then sit a multiple of 256 bytes apart).
    static constexpr int AS = BK + 8;
    static constexpr int BS = BN;
    static constexpr int A_STAGE = BM * AS;
    static constexpr int B_STAGE = BK * BS;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_BYTES = NBUF * STAGE * 4;
    static constexpr int A_VEC = BM * BK / 4 / NT;   // 16-byte loads per thread per stage
    static constexpr int B_VEC = BK * BN / 4 / NT;
    static constexpr int A_PART = (RB + 3) / 4;      // A fragments fetched per sub-step
    static_assert(BM % WM == 0 && BN % WN == 0, "wave grid must tile the block");
    static_assert(WM % 16 == 0 && WN % 64 == 0, "wave tile: 16-row x 64-column units");
    static_assert(BK % 16 == 0, "K step is a multiple of 16");
    static_assert(NBUF == 2 || NBUF == 3, "two or three LDS stages");
    static_assert(A_VEC * NT * 4 == BM * BK && B_VEC * NT * 4 == BK * BN,
                  "tile loads must divide evenly over the workgroup");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
};

// Load one 4-float chunk of A starting at (row gm, column gk).  GUARD: zero
// outside [0,M) x [0,K), without divergent branches in the common case: the
// address is clamped to the matrix start and the value selected.  VEC: one
// 16-byte load when the chunk is whole; only a chunk straddling K is read
// element by element.
template <bool GUARD, bool VEC>
__device__ __forceinline__ floatx4 load_a(const Problem &p, int gm, int gk) {
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

// Load one 4-float chunk of B starting at (row gk, column gn); as load_a.
template <bool GUARD, bool VEC>
__device__ __forceinline__ floatx4 load_b(const Problem &p, int gk, int gn) {
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

template <class S, bool GUARD, bool VEC>
__device__ __forceinline__ void global_to_regs(const Problem &p, int m0, int n0, int k0, int tid,
                                               floatx4 (&ra)[S::A_VEC], floatx4 (&rb)[S::B_VEC]) {
    constexpr int BK = S::KC * 16, BN = S::BS;
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

template <class S>
__device__ __forceinline__ void regs_to_lds(float *stage, int tid, const floatx4 (&ra)[S::A_VEC],
                                            const floatx4 (&rb)[S::B_VEC]) {
    constexpr int BK = S::KC * 16, BN = S::BS;
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

// A wave's operands.  For lane (i, g) and a 16-wide k-chunk, a[rb] holds
// A(row 16rb + i, k = 4g + 0..3) -- the A operand of all four MFMA steps of
// the chunk in one 16-byte LDS read -- and, for MFMA step s, b[cg] holds
// B(k = 4g + s, columns 64cg + 4i + 0..3), the B operand of the four column
// blocks of group cg.
template <class S>
struct AFrag {
    floatx4 a[S::RB];
};
template <class S>
struct BFrag {
    floatx4 b[S::CG];
};

// Quarter `part` of the A fragments of chunk `kc`.  Splitting them lets the
// next chunk's A be read between the MFMA steps of the current one.
template <class S>
__device__ __forceinline__ void load_a_part(const float *stage, int kc, int part, int lane, int wr,
                                            AFrag<S> &f) {
    const float *As = stage + (wr * (S::RB * 16) + (lane & 15)) * S::AS + 4 * (lane >> 4) + kc * 16;
#pragma unroll
    for (int q = 0; q < S::A_PART; ++q) {
        const int rb = part * S::A_PART + q;
        if (rb < S::RB) f.a[rb] = *reinterpret_cast<const floatx4 *>(As + rb * 16 * S::AS);
    }
}

template <class S>
__device__ __forceinline__ void load_b_step(const float *stage, int kc, int s, int lane, int wc,
                                            BFrag<S> &f) {
    const float *Bs = stage + S::A_STAGE + (kc * 16 + 4 * (lane >> 4) + s) * S::BS +
                      wc * (S::CG * 64) + 4 * (lane & 15);
#pragma unroll
    for (int cg = 0; cg < S::CG; ++cg) f.b[cg] = *reinterpret_cast<const floatx4 *>(Bs + cg * 64);
}

// MFMA step s of a chunk: RB x CG x 4 independent 16x16x4 products.
template <class S>
__device__ __forceinline__ void mfma_step(const AFrag<S> &fa, const BFrag<S> &fb, int s,
                                          floatx4 (&acc)[S::RB][S::CG * 4]) {
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
        for (int cg = 0; cg < S::CG; ++cg)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[rb][cg * 4 + c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                    fa.a[rb][s], fb.b[cg][c], acc[rb][cg * 4 + c], 0, 0, 0);
}

// alpha/beta epilogue and stores.  beta == 0 never reads C.
template <class S, bool GUARD, bool VEC>
__device__ __forceinline__ void store_tile(const Problem &p, int row0, int col0, int lane,
                                           const floatx4 (&acc)[S::RB][S::CG * 4]) {
    const int i = lane & 15, g = lane >> 4;
    const bool read_c = (p.beta != 0.f);
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int gm = row0 + rb * 16 + 4 * g + r;
            if (GUARD && gm >= p.M) continue;
            float *crow = p.C + (long long)gm * p.ldc;
#pragma unroll
            for (int cg = 0; cg < S::CG; ++cg) {
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

// Pipeline (per workgroup; t = K stage, NBUF = 2 or 3 LDS buffers):
//   * global loads of stage t + NBUF - 1 are issued at the top of stage t and
//     written to LDS buffer (t + NBUF - 1) % NBUF in the middle of stage t's
//     last chunk.  That buffer was last read during stage t - 1, which every
//     wave finished before the barrier that closed it, so the write is safe.
//   * the fragments of the next 16-wide chunk are read from LDS in four parts
//     between the MFMA steps of the current chunk.  With three buffers the
//     next stage's buffer is complete before stage t begins, so its first
//     chunk is prefetched before the barrier that closes stage t and no LDS
//     latency is exposed after it; with two it is read after the barrier.
//   * one barrier per stage.
// Scheduling fences between MFMA steps keep the compiler from hoisting every
// LDS read of the stage to its top (which would exhaust the registers).
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int OCC, bool VEC>
__global__ void __launch_bounds__((MfmaShape<BM, BN, BK, WM, WN, NBUF, OCC>::NT), OCC)
mfma_sgemm_kernel(Problem p, int tiles_m, int tiles_n, int group_m) {
    using S = MfmaShape<BM, BN, BK, WM, WN, NBUF, OCC>;
    __shared__ __attribute__((aligned(16))) float smem[NBUF * S::STAGE];
    select_batch(p);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wr = wave / S::WAVES_N, wc = wave % S::WAVES_N;

    int tm, tn;
    tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const bool interior = (m0 + BM <= p.M) && (n0 + BN <= p.N);

    floatx4 acc[S::RB][S::CG * 4];
#pragma unroll
    for (int a = 0; a < S::RB; ++a)
#pragma unroll
        for (int b = 0; b < S::CG * 4; ++b) acc[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};

    floatx4 ra[S::A_VEC], rb[S::B_VEC];
    const int nk = (p.K + BK - 1) / BK;

    auto fetch = [&](int t) {
        const int k0 = t * BK;
        if (interior && k0 + BK <= p.K)
            global_to_regs<S, false, VEC>(p, m0, n0, k0, tid, ra, rb);
        else
            global_to_regs<S, true, VEC>(p, m0, n0, k0, tid, ra, rb);
    };

    // prologue: stages 0 .. NBUF-2 into LDS
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t) {
        if (t < nk) {
            fetch(t);
            regs_to_lds<S>(smem + t * S::STAGE, tid, ra, rb);
        }
    }
    __syncthreads();

    AFrag<S> a_cur, a_nxt;
    BFrag<S> b_cur, b_nxt;
#pragma unroll
    for (int q = 0; q < 4; ++q) load_a_part<S>(smem, 0, q, lane, wr, a_cur);
    load_b_step<S>(smem, 0, 0, lane, wc, b_cur);

    for (int t = 0; t < nk; ++t) {
        const float *sb = smem + (t % NBUF) * S::STAGE;
        const int tf = t + NBUF - 1;             // stage fetched during this one
        const bool fetching = tf < nk;
        if (fetching) fetch(tf);
        const bool next_stage = (NBUF == 3) && (t + 1 < nk);
        const float *nsb = smem + ((t + 1) % NBUF) * S::STAGE;
#pragma unroll
        for (int kc = 0; kc < S::KC; ++kc) {
            const bool last = (kc == S::KC - 1);
            const bool next_chunk = !last || next_stage;   // operands of a following chunk readable now
            const float *csb = last ? nsb : sb;            // stage holding the following chunk
            const int ckc = last ? 0 : kc + 1;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < 3)
                    load_b_step<S>(sb, kc, s + 1, lane, wc, b_nxt);
                else if (next_chunk)
                    load_b_step<S>(csb, ckc, 0, lane, wc, b_nxt);
                if (next_chunk) load_a_part<S>(csb, ckc, s, lane, wr, a_nxt);
                mfma_step<S>(a_cur, b_cur, s, acc);
                if (last && s == 1 && fetching)
                    regs_to_lds<S>(smem + (tf % NBUF) * S::STAGE, tid, ra, rb);
                pipeline_fence();
                if (s < 3 || next_chunk) b_cur = b_nxt;
            }
            if (next_chunk) a_cur = a_nxt;
        }
        __syncthreads();
        if (NBUF == 2 && t + 1 < nk) {
#pragma unroll
            for (int q = 0; q < 4; ++q) load_a_part<S>(nsb, 0, q, lane, wr, a_cur);
            load_b_step<S>(nsb, 0, 0, lane, wc, b_cur);
        }
    }

    const int row0 = m0 + wr * WM, col0 = n0 + wc * WN;
    if (interior)
        store_tile<S, false, VEC>(p, row0, col0, lane, acc);
    else
        store_tile<S, true, VEC>(p, row0, col0, lane, acc);
}

template <int BM, int BN, int BK, int WM, int WN, int NBUF, int OCC, bool VEC>
hipError_t launch_mfma(const Problem &p, int group_m, hipStream_t stream) {
    using S = MfmaShape<BM, BN, BK, WM, WN, NBUF, OCC>;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    const long long tiles = (long long)tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (group_m <= 0) group_m = 4;
    hipLaunchKernelGGL((mfma_sgemm_kernel<BM, BN, BK, WM, WN, NBUF, OCC, VEC>),
                       dim3((unsigned)tiles, p.batch), dim3(S::NT), 0, stream, p, tiles_m, tiles_n,
                       group_m);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int NBUF, int OCC>
constexpr TileEntry mfma_entry(int eff_pct) {
    using S = MfmaShape<BM, BN, BK, WM, WN, NBUF, OCC>;
    return TileEntry{{BM, BN, BK, WM, WN, 0, 0, S::NT, S::LDS_BYTES, NBUF, 0},
                     &launch_mfma<BM, BN, BK, WM, WN, NBUF, OCC, true>,
                     &launch_mfma<BM, BN, BK, WM, WN, NBUF, OCC, false>, eff_pct};
}

}  // namespace

// Compiled tile configurations (index = sgemm_config.tile for the MFMA family).
const TileEntry *mfma_tiles(int *count) {
    static const TileEntry tiles[] = {
        // argument: % of the fp32 peak measured at 4096^3
        mfma_entry<256, 256, 16, 128, 128, 3, 1>(80),   // 0: 4 waves, 256 accumulators per lane
        mfma_entry<256, 256, 16, 128, 128, 2, 1>(83),   // 1
        mfma_entry<256, 256, 32, 128, 128, 2, 1>(84),   // 2
        mfma_entry<256, 128, 16, 128, 64, 3, 1>(75),    // 3: 4 waves, 128 accumulators per lane
        mfma_entry<128, 128, 16, 64, 64, 3, 2>(81),     // 4: 2 waves per SIMD
        mfma_entry<128, 128, 32, 64, 64, 2, 2>(82),     // 5
        mfma_entry<128, 64, 32, 64, 64, 2, 1>(75),      // 6: 2 waves (1 per SIMD: registers)
        mfma_entry<64, 64, 32, 32, 64, 2, 2>(75),       // 7: small problems
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

}  // namespace sg
