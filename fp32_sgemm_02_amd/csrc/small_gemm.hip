// small_gemm.hip -- products whose C holds too few 64 x 64 tiles to occupy the
// chip's 256 CUs (256^3 is 16 such tiles; C of 777 x 777 with K = 33 is 169,
// each with two k-steps of work), so that the tiled families leave most CUs
// idle and pay their pipeline start-up on every tile.
//
// Each wave computes one 16 x 16*CB block of C on the matrix cores
// (v_mfma_f32_16x16x4_f32) from operands loaded straight from memory into
// registers: a block's operands are used by that wave only, so there is no
// LDS staging and no barrier in the k-loop ("a CUDA matmul" section 02: one
// thread per output cell, here one wave per 16x16 block; at these sizes the
// operands come from L2).  A workgroup holds WTM x WTN blocks times KW
// k-groups: the KW waves of a block take contiguous shares of K and their sums
// meet in LDS in a fixed order at the end.  Small blocks and k-groups
// multiply the waves a small product keeps busy: 256^3 in 16 x 64 blocks with
// four k-groups is 64 workgroups of 4 waves, in 16 x 16 blocks 256.
//
// Operands of lane l (i = l % 16, g = l / 16) in the 16-wide k-chunk at k0:
// MFMA step s (0..3) of the chunk takes k = k0 + 4g + s; the A operand is
// A(row i of the block, k), the B operand of column block cb is B(k, column
// c(i)), where c(i) = i for CB == 1 and 4i + cb for CB == 4 (lane i then
// holds four adjacent columns of each row and stores them 16 bytes at a
// time).  Result register r of block cb is C(row 4g + r, column c(i)).  A
// k-contiguous operand (A, or B stored transposed) gives a lane its four k
// values with one 16-byte load (four 4-byte loads when rows are not 16-byte
// aligned); B untransposed gives them from four rows, 16 bytes each for
// CB == 4 (one per step, feeding the four column blocks) or 4 bytes each
// for CB == 1.
//
// Every load is a buffer load whose offset is chosen without a branch: a lane
// whose element lies outside the matrix or outside its k-group's share gets an
// offset past the buffer's range and reads zero ("The 1% kernel" section 6:
// idle threads past the matrix).  A per-lane branch around a load would make
// the compiler wait for all loads in flight at the join.
#include <cstdint>

#include "gemm_internal.hpp"

namespace sg {
namespace {

constexpr int kOff = (int)0x80000000u;   // past every resource's range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t small_rsrc(const float *base, long long bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ floatx4 sld4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float sld1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

template <int CB, int WTM, int WTN, int KW, int U>
struct SmallShape {
    static_assert(CB == 1 || CB == 4, "one or four 16-column blocks per wave");
    static constexpr int BLOCKS = WTM * WTN;       // blocks of C per workgroup
    static constexpr int NW = BLOCKS * KW;         // waves
    static constexpr int NT = 64 * NW;
    static constexpr int BM = 16 * WTM, BN = 16 * CB * WTN;
    static constexpr int NBV = CB == 1 ? 1 : 4;    // B vectors per chunk and lane
    // partial sums of k-groups 1.. (floatx4 per lane and column block)
    static constexpr int RED = (KW - 1) * BLOCKS * CB * 64;
    static constexpr int LDS_BYTES = RED * 16;
    static_assert(NT <= 1024, "workgroup size");
};

// The operands of U consecutive chunks.  a[u]: this lane's four k values of
// its A row.  b[u][v]: for B stored transposed or CB == 1, v = column block
// and the four k values; for B untransposed with CB == 4, v = step s and the
// four adjacent columns 4i .. 4i+3.
template <int CB, int U>
struct SmallRound {
    floatx4 a[U];
    floatx4 b[U][CB == 1 ? 1 : 4];
};

template <int CB, bool TB>
__device__ __forceinline__ float b_op(const floatx4 (&b)[CB == 1 ? 1 : 4], int s, int cb) {
    if constexpr (CB == 1)
        return b[0][s];
    else if constexpr (TB)
        return b[cb][s];
    else
        return b[s][cb];
}

// Loads of chunks c .. c+U-1.  row: this lane's row of A (m0 + i); cols:
// first column of its B vector(s).  kend: end of this k-group's share.
template <int CB, int U, bool TB, bool VA, bool VB>
__device__ __forceinline__ void small_load(const Problem &p, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int row, int col, int g,
                                           int c, int kend, SmallRound<CB, U> &r) {
    const bool row_ok = row < p.M;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = 16 * (c + u) + 4 * g;
        if constexpr (VA) {
            // K % 4 == 0, so the four k values are inside or outside together
            r.a[u] = sld4(ra, (row_ok && k < kend) ? (int)((row * p.lda + k) * 4) : kOff);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                r.a[u][s] = sld1(ra, (row_ok && k + s < kend) ? (int)((row * p.lda + k + s) * 4)
                                                              : kOff);
        }
        if constexpr (TB) {
            // row n of B^T holds column n; CB == 4: column block cb is column 4i + cb
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int n = col + cb;
                const bool ok = n < p.N;
                if constexpr (VB) {
                    r.b[u][cb] = sld4(rb, (ok && k < kend) ? (int)((n * p.ldb + k) * 4) : kOff);
                } else {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        r.b[u][cb][s] =
                            sld1(rb, (ok && k + s < kend) ? (int)((n * p.ldb + k + s) * 4) : kOff);
                }
            }
        } else if constexpr (CB == 1) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                r.b[u][0][s] = sld1(rb, (col < p.N && k + s < kend)
                                            ? (int)(((k + s) * p.ldb + col) * 4) : kOff);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if constexpr (VB) {
                    // N % 4 == 0: the four columns are inside or outside together
                    r.b[u][s] = sld4(rb, (col < p.N && k + s < kend)
                                             ? (int)(((k + s) * p.ldb + col) * 4) : kOff);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        r.b[u][s][e] = sld1(rb, (col + e < p.N && k + s < kend)
                                                    ? (int)(((k + s) * p.ldb + col + e) * 4)
                                                    : kOff);
                }
            }
        }
    }
}

template <int CB, int U, bool TB>
__device__ __forceinline__ void small_mma(const SmallRound<CB, U> &r, floatx4 (&acc)[CB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.a[u][s], b_op<CB, TB>(r.b[u], s, cb),
                                                               acc[cb], 0, 0, 0);
}

// alpha * sum (+ beta * C) (+ bias, activation) of one cell.
__device__ __forceinline__ float small_finish(const Problem &p, float old, int col, float sum) {
    float out = p.alpha * sum;
    if (p.beta != 0.f) out = fmaf(p.beta, old, out);
    if (p.has_epilogue()) out = activate(p.act, p.bias ? out + p.bias[col] : out);
    return out;
}

template <int CB, int WTM, int WTN, int KW, int U, bool TB, bool VA, bool VB>
__global__ void __launch_bounds__(64 * WTM * WTN * KW)
small_kernel(Problem p, int tiles_n, int cvec) {
    using S = SmallShape<CB, WTM, WTN, KW, U>;
    select_batch(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kg = wave / S::BLOCKS, wv = wave % S::BLOCKS;
    const int wr = wv / WTN, wc = wv % WTN;
    const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tm * S::BM + 16 * wr, n0 = tn * S::BN + 16 * CB * wc;
    const int i = lane & 15, g = lane >> 4;
    const int row = m0 + i;
    const int col = n0 + (CB == 1 ? i : 4 * i);

    // this k-group's share of the 16-wide chunks
    const int nc = (p.K + 15) / 16;
    const int per = (nc + KW - 1) / KW;
    const int c0 = kg * per;
    const int c1 = min(nc, c0 + per);
    const int kend = min(p.K, 16 * c1);

    const long long a_rows = p.M, b_rows = TB ? p.N : p.K;
    const __amdgpu_buffer_rsrc_t ra = small_rsrc(p.A, a_rows * p.lda * 4);
    const __amdgpu_buffer_rsrc_t rb = small_rsrc(p.B, b_rows * p.ldb * 4);

    floatx4 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = floatx4{0.f, 0.f, 0.f, 0.f};

    // beta != 0: the cells of C this wave finishes, loaded before the k-loop
    // so that their latency overlaps it (k-group 0 only; other waves, cells
    // outside C and beta == 0 read nothing).  oldc[cb][r] is C(row 4g + r,
    // column c(i) of block cb).
    floatx4 oldc[CB];
    {
        const bool want = p.beta != 0.f && kg == 0;
        const __amdgpu_buffer_rsrc_t rc = small_rsrc(p.C, (long long)p.M * p.ldc * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int gm = m0 + 4 * g + r;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int gn = col + cb;
                oldc[cb][r] = sld1(rc, (want && gm < p.M && gn < p.N)
                                           ? (int)((gm * p.ldc + gn) * 4) : kOff);
            }
        }
    }

    // double-buffered rounds of U chunks.  Chunks past c1 read zeros without
    // touching memory, so the loads inside the loop are issued
    // unconditionally: a load under a branch would make the compiler wait for
    // every load in flight at the join, including the prefetch that should
    // overlap the MFMAs.  A share of at most one round (short K) takes its
    // one round alone, without the loop's two rounds of prefetch past it; the
    // branch is uniform and comes before any load is in flight.
    SmallRound<CB, U> r0, r1;
    if (c1 - c0 <= U) {
        small_load<CB, U, TB, VA, VB>(p, ra, rb, row, col, g, c0, kend, r0);
        small_mma<CB, U, TB>(r0, acc);
    } else {
        small_load<CB, U, TB, VA, VB>(p, ra, rb, row, col, g, c0, kend, r0);
        for (int c = c0; c < c1; c += 2 * U) {
            small_load<CB, U, TB, VA, VB>(p, ra, rb, row, col, g, c + U, kend, r1);
            small_mma<CB, U, TB>(r0, acc);
            pipeline_fence();
            small_load<CB, U, TB, VA, VB>(p, ra, rb, row, col, g, c + 2 * U, kend, r0);
            if (c + U < c1) small_mma<CB, U, TB>(r1, acc);
            pipeline_fence();
        }
    }

    // k-groups 1.. leave their sums in LDS; group 0 adds them in group order
    if constexpr (KW > 1) {
        __shared__ floatx4 red[S::RED];
        if (kg > 0) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                red[(((kg - 1) * S::BLOCKS + wv) * CB + cb) * 64 + lane] = acc[cb];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int q = 1; q < KW; ++q)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const floatx4 v = red[(((q - 1) * S::BLOCKS + wv) * CB + cb) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[cb][e] += v[e];
            }
    }

    // C: rows 4g + r of the block; columns c(i) of each column block
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int gm = m0 + 4 * g + r;
        if (gm >= p.M) continue;
        float *crow = p.C + (long long)gm * p.ldc;
        if constexpr (CB == 4) {
            if (cvec && col + 3 < p.N) {
                floatx4 v;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    v[cb] = small_finish(p, oldc[cb][r], col + cb, acc[cb][r]);
                *reinterpret_cast<floatx4 *>(crow + col) = v;
                continue;
            }
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const int gn = col + cb;
            if (gn >= p.N) continue;
            crow[gn] = small_finish(p, oldc[cb][r], gn, acc[cb][r]);
        }
    }
}

template <int CB, int WTM, int WTN, int KW, int U, bool TB, bool VA, bool VB>
hipError_t launch_small_as(const Problem &p, hipStream_t stream) {
    using S = SmallShape<CB, WTM, WTN, KW, U>;
    const int tiles_m = (p.M + S::BM - 1) / S::BM, tiles_n = (p.N + S::BN - 1) / S::BN;
    const long long blocks = (long long)tiles_m * tiles_n;
    if (blocks > 0x7fffffffLL || p.batch > kMaxBatchPerLaunch) return hipErrorInvalidValue;
    const int cvec = rows_aligned(p.C, p.ldc, p.stride_c, p.batch, 4) ? 1 : 0;
    hipLaunchKernelGGL((small_kernel<CB, WTM, WTN, KW, U, TB, VA, VB>),
                       dim3((unsigned)blocks, p.batch), dim3(S::NT), 0, stream, p, tiles_n, cvec);
    return hipGetLastError();
}

// 16-byte loads where an operand allows them (VEC launcher only): A when its
// rows are 16-byte aligned and K % 4 == 0; B transposed likewise; B
// untransposed (CB == 4) when its rows are aligned and N % 4 == 0.
template <int CB, int WTM, int WTN, int KW, int U, bool VEC>
hipError_t launch_small(const Problem &p, int, hipStream_t stream) {
    if (p.trans_a) return hipErrorInvalidValue;
    const bool va = VEC && p.K % 4 == 0 && rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4);
    const bool b_al = rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4);
    if (p.trans_b) {
        const bool vb = VEC && p.K % 4 == 0 && b_al;
        if (va && vb) return launch_small_as<CB, WTM, WTN, KW, U, true, true, true>(p, stream);
        return launch_small_as<CB, WTM, WTN, KW, U, true, false, false>(p, stream);
    }
    const bool vb = VEC && CB == 4 && p.N % 4 == 0 && b_al;
    if (va && (vb || CB == 1)) return launch_small_as<CB, WTM, WTN, KW, U, false, true, true>(p, stream);
    return launch_small_as<CB, WTM, WTN, KW, U, false, false, false>(p, stream);
}

template <int CB, int WTM, int WTN, int KW, int U>
constexpr TileEntry small_entry() {
    using S = SmallShape<CB, WTM, WTN, KW, U>;
    // the kernel applies a problem's bias / activation itself, so the 16-byte
    // launcher is also the fused one; desc.tm: k-groups per block
    return TileEntry{{S::BM, S::BN, 16 * U, 16, 16 * CB, KW, 0, S::NT, S::LDS_BYTES, 0,
                      SGEMM_TILE_TRANS_B},
                     &launch_small<CB, WTM, WTN, KW, U, true>,
                     &launch_small<CB, WTM, WTN, KW, U, false>, 0,
                     &launch_small<CB, WTM, WTN, KW, U, true>};
}

}  // namespace

// Tiles (CB, WTM, WTN, KW, U): block 16 x 16*CB, WTM x WTN blocks, KW k-groups.
const TileEntry *small_tiles(int *count) {
    static const TileEntry tiles[] = {
        small_entry<1, 1, 1, 4, 4>(),   // 0: 16 x 16, 4 k-groups
        small_entry<1, 2, 2, 1, 4>(),   // 1: 32 x 32, 4 blocks
        small_entry<4, 1, 1, 4, 2>(),   // 2: 16 x 64, 4 k-groups
        small_entry<4, 2, 1, 2, 2>(),   // 3: 32 x 64, 2 blocks x 2 k-groups
        small_entry<4, 4, 1, 1, 2>(),   // 4: 64 x 64, 4 blocks
        small_entry<1, 1, 1, 8, 4>(),   // 5: 16 x 16, 8 k-groups
        small_entry<4, 1, 1, 8, 2>(),   // 6: 16 x 64, 8 k-groups
        small_entry<4, 2, 2, 1, 2>(),   // 7: 32 x 128, 4 blocks
    };
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

// The 32-bit buffer offsets must stay below 2^31 bytes: M * lda and the
// stored rows of B times ldb below 2^29 floats.  A stored transposed is not
// served.
bool small_fits(const Problem &p) {
    constexpr long long lim = 1LL << 29;
    return !p.trans_a && (long long)p.M * p.lda < lim &&
           (long long)(p.trans_b ? p.N : p.K) * p.ldb < lim;
}

// The family's tile for a problem (measured, graph-replayed, on MI355X over
// cubes 32..768, 777 x 777 x {33, 256}, 300 x 200 x 100, 256^2 x 4096,
// 128^2 x 8192 and 512^2 x 2048).  Blocks of 16 x 64 need B rows that take
// 16-byte loads (N % 4 == 0, or K % 4 == 0 for B stored transposed) and at
// least 64 columns; otherwise 16 x 16 blocks.  Long K over few blocks: the
// 16 x 16 blocks with 4 or 8 k-groups (more waves, L2-bound).  A few k-steps:
// no k-groups (32 x 32, 32 x 128 or 64 x 64 workgroup tiles).  Otherwise four
// k-groups, over 16 x 16 blocks while there are few 16 x 64 ones (256^3:
// 3.99 us against 4.64), else over 16 x 64 blocks.
int small_choice(const Problem &p) {
    const long long nc = (p.K + 15) / 16;
    const bool rows16 = p.trans_b ? p.K % 4 == 0 : p.N % 4 == 0;   // B rows in 16-byte loads
    const bool wide = p.N >= 64 && rows16;
    const long long b16 = (long long)((p.M + 15) / 16) * ((p.N + 15) / 16) * p.batch;
    const long long b64 = (long long)((p.M + 15) / 16) * ((p.N + 63) / 64) * p.batch;
    // very long K on a thin product (M or N at most 64) with more than a few
    // blocks: 16 x 64 blocks of eight k-groups while they are at most one per
    // CU (64 x 4096 x 4096 25.7 us, four k-groups 27.9; 4096 x 48 x 8192
    // 46.0, 16 x 16 blocks 89.8), else 32 x 64 workgroups of two k-groups (32
    // x 14336 x 4096 49.2 us against 67.5)
    if (rows16 && nc >= 256 && b64 > 64 && (p.M <= 64 || p.N <= 64))
        return b64 <= 256 ? 6 : 3;
    if (!wide) {
        if (nc >= 32 && b16 <= 512) return nc >= 64 && b16 <= 256 ? 5 : 0;
        return 1;
    }
    if (nc >= 64 && b64 <= 64) return nc >= 256 ? 5 : 0;
    if (nc <= 4) return b64 < 64 ? 1 : (p.M >= 32 && p.N >= 128 ? 7 : 4);
    return b64 <= 80 ? 0 : 2;
}

// Automatic dispatch: products with fewer than 256 tiles of 64 x 64 (the
// smallest tiled-family workgroup tile) across the batch -- or exactly 256 of
// them with K <= 64 (1000 x 1000 x 64: 5.9 us against 7.6) -- A
// untransposed, and at most 1.5 GFLOP.  Without reuse through LDS the family
// is bound by L2 bandwidth at a few tens of TFLOP/s, so larger products with
// few tiles (long K) go to stream-K (768 x 768 x 65536: 0.64 ms there) --
// except narrow ones (M or N at most 200) whose C covers less than 200
// tiles of 64 x 64 in area: they leave most CUs, or most rows or columns of
// the tiled families' tiles and of stream-K's 256-row tiles, idle.  64 x
// 4096 x 4096 25.7 us here against 72.8 for the best tiled plan, 33 x 2048 x
// 8192 42.1 against 90.2, 32 x 14336 x 4096 49.2 against 80.9, 3000 x 100
// x 3000 36.6 against 60.9, 192 x 4096 x 4096 66.5 against 75.3; 64 x 14336
// x 4096 (224 full tiles) stays tiled (76.7 us against 85.3).
//
// Batches of tiny products (each at most 64 x 64 and half that in area, K <=
// 512) take the family whatever their count: a tiled-family workgroup would
// leave most of its tile idle, and the few-rows kernel is built for long
// rows of B.  Graph-replayed: 4096 x 32^3 18.3 us against 22.7 (the 64 x 64
// k-group tile), 2048 x 16 x 64 x 128 with B^T 19.3 against 31.8 (few rows);
// 1024 x 64^3 stays on the tiled family (9.2 us against 13.8).
bool small_tiny_batch(const Problem &p) {
    return p.batch > 1 && p.M <= 64 && p.N <= 64 && (long long)p.M * p.N <= 2048 && p.K <= 512;
}

int small_pick(const Problem &p) {
    if (!small_fits(p)) return -1;
    const long long t64 = (long long)((p.M + 63) / 64) * ((p.N + 63) / 64) * p.batch;
    const double flops = 2.0 * p.M * p.N * (double)p.K * p.batch;
    const bool few = t64 < 256 || (t64 == 256 && p.K <= 64);
    const bool narrow = (p.M <= 200 || p.N <= 200) && (long long)p.M * p.N < 200LL * 64 * 64;
    return ((few && (flops <= 1.5e9 || narrow)) || (small_tiny_batch(p) && flops <= 1.5e9))
               ? small_choice(p)
               : -1;
}

}  // namespace sg
