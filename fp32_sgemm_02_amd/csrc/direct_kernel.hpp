// direct_kernel.hpp -- fp32 SGEMM on the matrix cores with global -> LDS
// direct loads (the kernel templates; mfma_direct.hip and mfma_direct_ta.hip
// instantiate them as tile tables).
//
// Same operation and the same tiling hierarchy as mfma_gemm.hip (workgroup
// tiles of C, K-slices staged in LDS and reused, wave tiles computed as sums
// of 16x16x4 outer-product blocks -- "The GEMM Scrapbook", shared-memory,
// 2D-tiling and warptiling chapters; "a CUDA matmul" section 05), with three
// changes to how a K-slice reaches LDS:
//   * it is copied by buffer_load_dwordx4 ... lds: the memory pipeline writes
//     each lane's 16 bytes straight into LDS, so the slice occupies no
//     registers and costs no LDS-write instructions (on gfx950 a burst of
//     ds_write_b128 per stage stalled the single wave of each SIMD for
//     ~1,100 cycles);
//   * the LDS image is unpadded: lane l of a load lands at byte 16*l of its
//     1 KB block.  Bank conflicts on the A-fragment reads are avoided by an
//     XOR swizzle instead of padding: the 16-byte chunk c of A-tile row r is
//     stored in slot c ^ ((r >> 1) & (BK/4 - 1)) (kswz below), a pattern measured
//     conflict-free for the 16-row x 4-chunk reads of a wave ("The GEMM
//     Scrapbook", warptiling chapter: arrange accesses so the lanes hit
//     distinct banks);
//   * the barrier that publishes stage t+1 sits in the middle of stage t,
//     and every LDS read and load issue of a stage is spread between its
//     MFMAs (rolling fragments, below) instead of queueing at its end.
// Used only when A, B, C are 16-byte aligned with leading dimensions that are
// multiples of 4 and M, N, K are multiples of BM, BN, BK: no guards.
//
// Register budget: a wave tile of 128x64 (or 64x128) keeps 128 accumulators
// per lane, which the compiler holds in place; with 128x128 wave tiles (256
// accumulators) it shuffled accumulators between register files on every
// K-step.  So the 256x256 tiles run 8 waves, two per SIMD, and the second
// wave of a SIMD covers the LDS latency of the first.
//
// Rolling fragments.  The MFMAs of a stage run row block by row block (all
// four k-steps of 16-row block rb, then rb+1), so A fragment a[rb] is dead as
// soon as its block is done and its registers take the next stage's a[rb];
// only the B fragments need a second set.  With RB row blocks per wave and
// H = RB/2, per workgroup (NBUF LDS buffers, stage t in buffer t % NBUF):
//   prologue     issue stages 0 .. NBUF-1; wait for stage 0; barrier; read
//                a[0 .. H-1] and B of stage 0
//   stage t      blocks 0 .. H-1: before block rb, read a[H + rb] of stage t
//                wait until this wave's loads of stage t+1 have landed;
//                barrier (stage t+1 is then complete for every wave, and no
//                wave reads stage t's buffer any more)
//                blocks H .. RB-1: before block rb, read the next stage's
//                a[rb - H] and a share of its B fragments, and issue a share
//                of the loads of stage t+NBUF into buffer t % NBUF
// A load issued in stage t is waited for in the middle of stage t+NBUF-1.
#pragma once

#include <cstdint>
#include <type_traits>

#include "gemm_internal.hpp"

namespace sg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
}  // namespace

bool direct_applies(const Problem &p, int bm, int bn, int bk, bool edges);

namespace {

// AV, BV: floats per direct load of A and B (4: buffer_load_dwordx4, needs
// 16-byte aligned rows; 1: buffer_load_dword, any 4-byte aligned layout;
// 5: buffer_load_dwordx4 from rows that are only 4-byte aligned, with the
// k-tail stage taken by dword loads -- k-contiguous operands only, i.e. A
// untransposed and B transposed).  A 16-byte load needs no 16-byte alignment
// on gfx9-family parts run by the ROCm driver (unaligned access mode; the
// compiler emits such loads itself for 4-byte aligned 16-byte data).  What it
// cannot do is stop at the K bound inside a chunk: on the last stage a chunk
// may straddle K, and there each float is loaded alone so that those past K
// read zeros.
// KG: k-groups.  With KG > 1 the waves form KG groups that each own the same
// BM x BN tile of C and take turns over the 16-wide k-chunks of a stage
// (group g: chunks g*KC/KG ..); their partial sums meet in LDS at the end.
// It multiplies the waves working on one tile, for problems whose tiles are
// too few or too small to keep every SIMD busy.
// TB: B is stored transposed (N x K, k contiguous, ldb >= K); its tile is then
// held in LDS like A's (BN rows of BK floats, same swizzle), with the rows of
// each 64-column group permuted so that lane i's four column blocks are four
// adjacent columns, as for untransposed B (16-byte stores of C).
// TA: A is stored transposed (K x M, m contiguous, lda >= M); its tile is held
// in LDS like untransposed B's (BK rows of BM floats, unswizzled) and read the
// same way: one 16-byte read gives four 16-row blocks their operand of one
// MFMA step, so the rows of a 64-row group are interleaved (row 4i + c of
// the group is row i of block c).
// EP: the instance applies the fused epilogue (no effect on the shape; it
// keeps the shape types of the two instances apart).
// IN: input format, 0 fp32; 1 bfloat16, 2 float16 (16-bit inputs, fp32
// accumulation): A and B^T are then read as matrices of 32-bit words, each
// word two adjacent k values, so every size along k below (BK, K, lda, ldb,
// the 16-byte chunks) counts words, the LDS image and its loads are those of
// the fp32 kernel, and a lane's 16-byte fragment is the 8 k values of one
// v_mfma_f32_16x16x32 instead of the 4 k-steps of v_mfma_f32_16x16x4.  Only
// k-contiguous operands (A untransposed, B transposed) have that word form.
// MD: the kernel's mode (0 one tile per workgroup, 1 stream-K runs, 2
// stream-K fixup); like EP it only keeps the shape types of instances apart.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int AV = 4, int BV = 4, int KG = 1,
          bool TB = false, bool TA = false, bool EP = false, int IN = 0, int MD = 0>
struct DirectShape {
    static constexpr int WAVES_M = BM / WM;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int WAVES_MN = WAVES_M * WAVES_N;  // waves of one k-group
    static constexpr int NW = WAVES_MN * KG;
    static constexpr int NT = NW * 64;
    static constexpr int RB = WM / 16;
    static constexpr int CG = WN / 64;
    static constexpr int CB = WN / 16;                  // 16-column blocks of a wave tile
    static constexpr bool TRANS_B = TB;
    static constexpr bool TRANS_A = TA;
    static constexpr int INPUT = IN;
    static_assert(IN == 0 || (TB && !TA), "16-bit inputs: A untransposed, B transposed");
    static_assert(!TA || WM % 64 == 0, "transposed A: 64-row groups per wave");
    static constexpr int CPR_A = BK / 4;                // 16-byte chunks per A-tile row
    static constexpr int CPR_B = BN / 4;                // ... per B-tile row
    static constexpr int A_STAGE = BM * BK;             // floats
    static constexpr int B_STAGE = BK * BN;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_BYTES = NBUF * STAGE * 4;
    static constexpr int AVEC = AV == 1 ? 1 : 4, BVEC = BV == 1 ? 1 : 4;   // floats per load
    static constexpr bool A_SPLIT = AV == 5, B_SPLIT = BV == 5;   // dword loads on the k tail
    static constexpr int LA = A_STAGE / AVEC / 64 / NW;   // direct loads per wave per stage (A)
    static constexpr int LB = B_STAGE / BVEC / 64 / NW;   // ... (B)
    static constexpr int L = LA + LB;
    static constexpr int KC = BK / 16;                  // 16-wide k-chunks per stage
    static constexpr int KCW = KC / KG;                 // ... per wave
    static constexpr int RED_FLOATS = (KG - 1) * WAVES_MN * (WM / 16) * (WN / 64) * 16 * 64;
    static_assert(BK == 16 || BK == 32, "one or two 16-wide k-chunks per stage");
    static_assert(KG >= 1 && KC % KG == 0, "k-groups split the chunks of a stage evenly");
    static_assert(RED_FLOATS <= NBUF * STAGE, "k-group partial sums fit the LDS ring");
    static_assert(WM % 16 == 0 && WN % 64 == 0, "wave tile: 16-row x 64-column units");
    static_assert((AV == 4 || AV == 1 || AV == 5) && (BV == 4 || BV == 1 || BV == 5),
                  "dword or dwordx4 loads");
    static_assert(!A_SPLIT || !TA, "split tail loads need k-contiguous A rows");
    static_assert(!B_SPLIT || TB, "split tail loads need k-contiguous B rows");
    static_assert(LA * 64 * NW * AVEC == A_STAGE && LB * 64 * NW * BVEC == B_STAGE,
                  "stage loads divide evenly over the waves");
    static_assert(NBUF >= 2 && LDS_BYTES <= 160 * 1024, "LDS ring of 2+ stages");
    // the k-tail stage of a split operand issues 4 dword loads per 16-byte load
    static_assert(L * (NBUF - 1) + 3 * (A_SPLIT ? LA : 0) + 3 * (B_SPLIT ? LB : 0) <= 63,
                  "outstanding loads fit the vmcnt counter");
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct loads of one stage.  The A tile is BM rows of CPR_A 16-byte chunks
// stored row-major; the chunk in slot `slot` of row r holds logical chunk
// slot ^ swz(r) (kswz below).  Load j of a wave fills the
// next 64 * AV floats of the tile image (lane l writes floats AV*l .. +AV-1 of
// them), so each lane loads whatever global element(s) belong there.  The B
// slice (BK x BN, row-major, unswizzled) is filled the same way.
//
// With edges (GUARD), a lane whose element lies outside the matrix gets an
// offset past the buffer's range: the hardware then writes zeros into LDS
// without touching memory.  Rows past M and columns past N are fixed per
// lane; the k bound is applied on the last stage only.
constexpr int kOutOfRange = (int)0x80000000u;

// The swizzle of a k-contiguous tile image (A untransposed, B transposed):
// the 16-byte chunk c of row r sits in slot c ^ kswz(r).  It depends on the
// row within its 16-row block only (the fragment reads of an MFMA block take
// rows 16b + i, i = lane % 16, one logical chunk), and gives those 16 rows
// distinct banks: rows of 64 or 128 bytes (BK = 16, 32) share a 256-byte
// bank line four or two at a time, so the rows pair up as r >> 1.
template <class S>
__device__ __forceinline__ int kswz(int r) {
    static_assert(S::CPR_A == 4 || S::CPR_A == 8, "rows of 64 or 128 bytes");
    return (r >> 1) & (S::CPR_A - 1);
}

// Row r and k (within the stage) of float w of a k-contiguous tile image:
// rows of BK floats whose 16-byte chunks sit in swizzled slots (kswz).
template <class S>
__device__ __forceinline__ void kimage_pos(int w, int &r, int &k) {
    constexpr int BK = S::KC * 16;
    r = w / BK;
    const int kk = w % BK;
    k = 4 * ((kk / 4) ^ kswz<S>(r)) + kk % 4;
}

// Column of the tile held in LDS row r of a transposed-B image: row 64q +
// 16c + i holds column 64q + 4i + c, so that the 16-row block c of a
// 64-column group is columns 4i + c.
__device__ __forceinline__ int tb_column(int r) {
    return (r & ~63) | ((r & 15) << 2) | ((r >> 4) & 3);
}

template <class S>
struct DirectLanes {
    int a_off[S::LA];   // byte offsets within the A panel (row-major, lda)
    int b_off[S::LB];   // byte offsets within the B slice (row-major, ldb)
    int a_k[S::LA];     // k within the stage of each A load (its first element)
    int b_k[S::LB];     // k within the stage of each B load
};

template <class S, bool GUARD>
__device__ __forceinline__ DirectLanes<S> direct_lanes(const Problem &p, int m0, int n0, int wave,
                                                       int lane) {
    DirectLanes<S> d;
#pragma unroll
    for (int j = 0; j < S::LA; ++j) {
        const int w = (wave * S::LA + j) * 64 * S::AVEC + S::AVEC * lane;   // float in the tile
        if constexpr (S::TRANS_A) {
            // BK rows (k) of BM floats, like untransposed B
            constexpr int BMT = S::RB * 16 * S::WAVES_M;
            const int r = w / BMT, m = w % BMT;
            d.a_k[j] = r;
            d.a_off[j] = (GUARD && m0 + m >= p.M) ? kOutOfRange : (r * (int)p.lda + m) * 4;
        } else {
            int r, k;
            kimage_pos<S>(w, r, k);
            d.a_k[j] = k;
            d.a_off[j] = (GUARD && m0 + r >= p.M) ? kOutOfRange : (r * (int)p.lda + k) * 4;
        }
    }
#pragma unroll
    for (int j = 0; j < S::LB; ++j) {
        const int w = (wave * S::LB + j) * 64 * S::BVEC + S::BVEC * lane;
        if constexpr (S::TRANS_B) {
            // BN rows of BK floats, swizzled like A, rows permuted (tb_column)
            int r, k;
            kimage_pos<S>(w, r, k);
            const int n = tb_column(r);
            d.b_k[j] = k;
            d.b_off[j] = (GUARD && n0 + n >= p.N) ? kOutOfRange : (n * (int)p.ldb + k) * 4;
        } else {
            const int r = w / (S::CPR_B * 4), n = w % (S::CPR_B * 4);
            d.b_k[j] = r;
            d.b_off[j] = (GUARD && n0 + n >= p.N) ? kOutOfRange : (r * (int)p.ldb + n) * 4;
        }
    }
    return d;
}

// Loads [lo, hi) of stage t (index < LA: A loads, else B loads).
template <class S, bool GUARD>
__device__ __forceinline__ void issue_stage(const Problem &p, int m0, int n0, int t, float *buf,
                                            int wave, const DirectLanes<S> &d, int lo, int hi) {
    constexpr int BK = S::KC * 16;
    const __amdgpu_buffer_rsrc_t ra =
        S::TRANS_A ? __builtin_amdgcn_make_buffer_rsrc(
                         (void *)(p.A + (long long)t * BK * p.lda + m0), (short)0,
                         (int)(BK * p.lda * 4), 0x00020000)
                   : __builtin_amdgcn_make_buffer_rsrc(
                         (void *)(p.A + (long long)m0 * p.lda + (long long)t * BK), (short)0,
                         (int)((S::RB * 16 * S::WAVES_M) * p.lda * 4), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        S::TRANS_B ? __builtin_amdgcn_make_buffer_rsrc(
                         (void *)(p.B + (long long)n0 * p.ldb + (long long)t * BK), (short)0,
                         (int)((S::CB * 16 * S::WAVES_N) * p.ldb * 4), 0x00020000)
                   : __builtin_amdgcn_make_buffer_rsrc(
                         (void *)(p.B + (long long)t * BK * p.ldb + n0), (short)0,
                         (int)(BK * p.ldb * 4), 0x00020000);
    const int krem = p.K - t * BK;   // k below this stays inside the matrix
    const bool tail = GUARD && krem < BK;
    static_assert(GUARD || !(S::A_SPLIT || S::B_SPLIT), "split tail loads are guarded");
#pragma unroll
    for (int q = 0; q < S::L; ++q) {
        if (q < lo || q >= hi) continue;
        if (q < S::LA) {
            float *dst = buf + (wave * S::LA + q) * 64 * S::AVEC;
            if constexpr (S::A_SPLIT) {
                if (tail) {
                    // the 256 floats of this load as four dword loads (lane l
                    // of load e fills float 64e + l), each checked against K
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        int r, k;
                        kimage_pos<S>((wave * S::LA + q) * 256 + 64 * e + (threadIdx.x & 63), r,
                                      k);
                        const int off = (k >= krem || m0 + r >= p.M) ? kOutOfRange
                                                                     : (r * (int)p.lda + k) * 4;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(dst + 64 * e),
                                                                 4, off, 0, 0, 0);
                    }
                    continue;
                }
            }
            const int off = (tail && d.a_k[q] >= krem) ? kOutOfRange : d.a_off[q];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)dst, 4 * S::AVEC, off, 0, 0,
                                                     0);
        } else {
            const int j = q - S::LA;
            float *dst = buf + S::A_STAGE + (wave * S::LB + j) * 64 * S::BVEC;
            if constexpr (S::B_SPLIT) {
                if (tail) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        int r, k;
                        kimage_pos<S>((wave * S::LB + j) * 256 + 64 * e + (threadIdx.x & 63), r,
                                      k);
                        const int n = tb_column(r);
                        const int off = (k >= krem || n0 + n >= p.N) ? kOutOfRange
                                                                     : (n * (int)p.ldb + k) * 4;
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(dst + 64 * e),
                                                                 4, off, 0, 0, 0);
                    }
                    continue;
                }
            }
            const int off = (tail && d.b_k[j] >= krem) ? kOutOfRange : d.b_off[j];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)dst, 4 * S::BVEC, off, 0, 0,
                                                     0);
        }
    }
}

// Fragment reads of k-chunk kc of a stage.  The MFMAs of a chunk run in RB
// units of 4*CB; unit u uses one A fragment, read just before it.  For lane
// (i, g):
//   A untransposed: unit u is row block u; a = A(row 16u + i, k = 16kc + 4g
//     + 0..3) (logical chunk 4kc + g of the row, stored in slot
//     (4kc + g) ^ swz);
//   A transposed: unit u is MFMA step s = u % 4 of the four row blocks of
//     row group u / 4; a = A(rows 64(u/4) + 4i + 0..3, k = 16kc + 4g + s).
// The B fragments of a chunk, v[]:
//   B untransposed: v[s * CG + cg] = B(k = 16kc + 4g + s, columns
//     64cg + 4i + 0..3), the B operand of MFMA step s for 4 column blocks;
//   B transposed:   v[cb] = B(k = 16kc + 4g + 0..3, column 64(cb/4) + 4i +
//     cb%4), read like A (LDS row 16cb + i holds that column), one 16-column
//     block for all four steps.
template <class S>
__device__ __forceinline__ void read_a(const float *buf, int kc, int rb, int lane, int wr,
                                       floatx4 &a) {
    const int i = lane & 15, g = lane >> 4;
    if constexpr (S::TRANS_A) {
        constexpr int BMT = S::RB * 16 * S::WAVES_M;
        a = *reinterpret_cast<const floatx4 *>(buf + (16 * kc + 4 * g + rb % 4) * BMT +
                                               wr * S::RB * 16 + (rb / 4) * 64 + 4 * i);
    } else {
        const int slot = (4 * kc + g) ^ kswz<S>(i);
        a = *reinterpret_cast<const floatx4 *>(
            buf + (wr * S::RB * 16 + rb * 16 + i) * (S::CPR_A * 4) + 4 * slot);
    }
}

template <class S>
struct BFrag {
    floatx4 v[4 * S::CG];
};

// Part `part` (0..3) of the B fragments of chunk kc: step `part` (B
// untransposed) or column blocks CG*part .. CG*part + CG-1 (transposed).
template <class S>
__device__ __forceinline__ void read_b_part(const float *buf, int kc, int part, int lane, int wc,
                                            BFrag<S> &b) {
    const int i = lane & 15, g = lane >> 4;
    if constexpr (S::TRANS_B) {
        const int slot = (4 * kc + g) ^ kswz<S>(i);
#pragma unroll
        for (int q = 0; q < S::CG; ++q) {
            const int cb = part * S::CG + q;
            b.v[cb] = *reinterpret_cast<const floatx4 *>(
                buf + S::A_STAGE + (wc * S::CB * 16 + cb * 16 + i) * (S::CPR_A * 4) + 4 * slot);
        }
    } else {
        const float *Bs = buf + S::A_STAGE + (16 * kc + 4 * g + part) * (S::CPR_B * 4) +
                          wc * S::CG * 64 + 4 * i;
#pragma unroll
        for (int cg = 0; cg < S::CG; ++cg)
            b.v[part * S::CG + cg] = *reinterpret_cast<const floatx4 *>(Bs + cg * 64);
    }
}

// B operand of MFMA step s for the wave's 16-column block cb.
template <class S>
__device__ __forceinline__ float b_operand(const BFrag<S> &b, int s, int cb) {
    if constexpr (S::TRANS_B)
        return b.v[cb][s];
    else
        return b.v[s * S::CG + cb / 4][cb % 4];
}

// The MFMAs of unit u over one k-chunk (4*CB of them).  acc[rb][cb] covers
// rows 16rb + i (A untransposed) or 64(rb/4) + 4i + rb%4 (transposed) of the
// wave tile, and columns 64(cb/4) + 4i + cb%4 (B either way), i = lane % 16:
// lane i holds four adjacent columns of a row, stored with one 16-byte write.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <class S>
__device__ __forceinline__ void roll_unit(int u, const floatx4 &a, const BFrag<S> &b,
                                          floatx4 (&acc)[S::RB][S::CB]) {
    if constexpr (S::INPUT == 1) {
        // 16-bit inputs: one MFMA per 16-column block covers the chunk's 32 k
#pragma unroll
        for (int cb = 0; cb < S::CB; ++cb)
            acc[u][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b.v[cb]), acc[u][cb], 0,
                0, 0);
    } else if constexpr (S::INPUT == 2) {
#pragma unroll
        for (int cb = 0; cb < S::CB; ++cb)
            acc[u][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b.v[cb]), acc[u][cb], 0,
                0, 0);
    } else if constexpr (S::TRANS_A) {
        const int s = u % 4, rg = u / 4;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int cb = 0; cb < S::CB; ++cb)
                acc[4 * rg + c][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                    a[c], b_operand<S>(b, s, cb), acc[4 * rg + c][cb], 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int cb = 0; cb < S::CB; ++cb)
                acc[u][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b_operand<S>(b, s, cb),
                                                                  acc[u][cb], 0, 0, 0);
    }
}

// Stream-K plan (MODE 1 and 2).  The first dp_tiles tiles (in tile order)
// are computed whole, tile g, g + groups, ... by workgroup g; the k-iterations
// (BK-wide stages) of the next sk_tiles tiles, iters each, are laid end to
// end and split into `groups` consecutive runs of per_wg, one per workgroup.
// A run's middle tiles are whole and stored directly; its first and last
// tile may be partial, and their un-scaled partial sums go to workspace slots
// 2g and 2g + 1 of run g (run g is taken by the workgroup that xcd_remap
// maps to g).  The fixup launch (MODE 2, one workgroup per
// split tile and row block of the waves) adds a tile's pieces in k order and
// stores C.  No workgroup waits for another.
struct StreamK {
    int dp_tiles = 0, sk_tiles = 0, iters = 0, per_wg = 0, groups = 0;
    float *ws = nullptr;
};

// Number of runs that touch stream-K tile `tl`.
__device__ __forceinline__ int sk_pieces(const StreamK &sk, int tl) {
    const long long first = (long long)tl * sk.iters, last = first + sk.iters - 1;
    return 1 + (int)(last / sk.per_wg - first / sk.per_wg);
}
// Workspace slot of the q-th run touching tile `tl`: the run of workgroup
// g = first / per_wg + q; the tile is g's first (slot 2g) unless g's run
// started in an earlier tile (slot 2g + 1, only possible for q == 0).
__device__ __forceinline__ int sk_slot(const StreamK &sk, int tl, int q) {
    const long long first = (long long)tl * sk.iters;
    const long long g = first / sk.per_wg + q;
    return (int)(2 * g + (g * sk.per_wg < first ? 1 : 0));
}

// GUARD: the problem has edges (M, N or K not tile multiples, or C not fit
// for 16-byte stores): zero-filled loads outside the matrix and guarded
// stores.  cvec: C rows allow 16-byte stores (used with GUARD only).  EPI:
// the epilogue adds p.bias and applies p.act.  MODE: 0 one tile per
// workgroup (blockIdx.x), 1 the stream-K runs, 2 the stream-K fixup.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int KG, bool TB, bool TA, int AV,
          int BV, bool GUARD, bool EPI = false, int IN = 0, int MODE = 0>
__global__ void __launch_bounds__((DirectShape<BM, BN, BK, WM, WN, NBUF, 4, 4, KG>::NT), 1)
mfma_direct_kernel(Problem p, int tiles_m, int tiles_n, int group_m, int cvec, StreamK sk) {
    using S = DirectShape<BM, BN, BK, WM, WN, NBUF, AV, BV, KG, TB, TA, EPI, IN, MODE>;
    constexpr int RB = S::RB, H = RB / 2;
    static_assert(RB % 2 == 0, "two halves of row blocks");
    static_assert(MODE == 0 || KG == 1, "stream-K tiles have one k-group");
    __shared__ __attribute__((aligned(1024))) float smem[NBUF * S::STAGE];
    select_batch(p);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kg = wave / S::WAVES_MN, wv = wave % S::WAVES_MN;   // k-group, wave within it
    const int wr = wv / S::WAVES_N, wc = wv % S::WAVES_N;
    const int kc0 = kg * S::KCW;                                 // this wave's first chunk
    const int nk = (p.K + BK - 1) / BK;

    floatx4 acc[RB][S::CB];
    auto zero_acc = [&]() {
#pragma unroll
        for (int x = 0; x < RB; ++x)
#pragma unroll
            for (int y = 0; y < S::CB; ++y) acc[x][y] = floatx4{0.f, 0.f, 0.f, 0.f};
    };
    floatx4 a[RB];
    BFrag<S> b0, b1;

    // The MFMAs of stages [tb, te) of the tile at (m0, n0), added to acc;
    // stage t sits in LDS buffer (t - tb) % NBUF.
    auto mainloop = [&](int m0, int n0, int tb, int te) {
        const DirectLanes<S> d = direct_lanes<S, GUARD>(p, m0, n0, wave, lane);
        // prologue: stages tb .. tb+NBUF-1 in flight; stage tb complete and published
#pragma unroll
        for (int i = 0; i < NBUF; ++i)
            if (tb + i < te)
                issue_stage<S, GUARD>(p, m0, n0, tb + i, smem + i * S::STAGE, wave, d, 0, S::L);
        if (te - tb >= NBUF)
            wait_vmcnt<(NBUF - 1) * S::L>();
        else
            wait_vmcnt<0>();
        __syncthreads();

#pragma unroll
        for (int rb = 0; rb < H; ++rb) read_a<S>(smem, kc0, rb, lane, wr, a[rb]);
#pragma unroll
        for (int s = 0; s < 4; ++s) read_b_part<S>(smem, kc0, s, lane, wc, b0);

        // One k-chunk: the MFMAs of this wave's chunk kc0 + kc of stage t with B
        // fragments bc, and the fragments of its following chunk (of this stage,
        // or its first chunk of the next) read into a[] and bn.  A wave's last
        // chunk of a stage holds the barrier and issues the loads of stage t+NBUF.
        auto chunk = [&](int t, int kcw, const BFrag<S> &bc, BFrag<S> &bn) {
            const float *cbuf = smem + ((t - tb) % NBUF) * S::STAGE;
            const bool last = (kcw == S::KCW - 1);
            const int kc = kc0 + kcw;
#pragma unroll
            for (int rb = 0; rb < H; ++rb) {
                read_a<S>(cbuf, kc, rb + H, lane, wr, a[rb + H]);
                roll_unit<S>(rb, a[rb], bc, acc);
                pipeline_fence();
            }
            const bool more = !last || (t + 1 < te);     // a following chunk exists
            const float *nbuf = cbuf;
            int nkc = kc + 1;
            if (last) {
                if (more) {
                    if (t + NBUF <= te)
                        wait_vmcnt<(NBUF - 2) * S::L>();
                    else
                        wait_vmcnt<0>();
                }
                __syncthreads();
                nbuf = smem + ((t + 1 - tb) % NBUF) * S::STAGE;
                nkc = kc0;
            }
            const int tf = t + NBUF;
            float *fbuf = smem + ((t - tb) % NBUF) * S::STAGE;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                if (more) {
                    read_a<S>(nbuf, nkc, j, lane, wr, a[j]);
#pragma unroll
                    for (int s = (4 * j) / H; s < (4 * (j + 1)) / H; ++s)
                        read_b_part<S>(nbuf, nkc, s, lane, wc, bn);
                }
                if (last && tf < te)
                    issue_stage<S, GUARD>(p, m0, n0, tf, fbuf, wave, d, (S::L * j) / H,
                                          (S::L * (j + 1)) / H);
                roll_unit<S>(H + j, a[H + j], bc, acc);
                pipeline_fence();
            }
        };
        if (S::KCW == 2) {
            // an even number of chunks per stage and wave: the B sets are back in place
            for (int t = tb; t < te; ++t) {
                chunk(t, 0, b0, b1);
                chunk(t, 1, b1, b0);
            }
        } else {
            // one chunk per stage and wave: two stages per iteration swap the B sets back
            int t = tb;
            for (; t + 1 < te; t += 2) {
                chunk(t, 0, b0, b1);
                chunk(t + 1, 0, b1, b0);
            }
            if (t < te) chunk(t, 0, b0, b1);
        }
    };

    // k-group reduction and the epilogue of the tile at (m0, n0): C from acc
    // finish(m0, n0, rlo, rhi): store row blocks [rlo, rhi) of every wave
    auto finish = [&](int m0, int n0, int rlo, int rhi) {
    // k-groups: groups 1.. leave their partial sums in LDS (the ring is free
    // once every wave has left the loop); group 0 adds them in group order
    // and writes C
    if constexpr (KG > 1) {
        constexpr int PER_WAVE = RB * S::CB;              // floatx4 per lane
        __syncthreads();
        if (kg > 0) {
            floatx4 *dst = reinterpret_cast<floatx4 *>(smem) +
                           ((kg - 1) * S::WAVES_MN + wv) * PER_WAVE * 64 + lane;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int j = 0; j < S::CB; ++j) dst[(rb * S::CB + j) * 64] = acc[rb][j];
        }
        __syncthreads();
        if (kg > 0) return;
#pragma unroll
        for (int g = 1; g < KG; ++g) {
            const floatx4 *src = reinterpret_cast<const floatx4 *>(smem) +
                                 ((g - 1) * S::WAVES_MN + wv) * PER_WAVE * 64 + lane;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int j = 0; j < S::CB; ++j) {
                    const floatx4 v = src[(rb * S::CB + j) * 64];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rb][j][e] += v[e];
                }
        }
    }

    // epilogue: alpha/beta (beta == 0 never reads C); 16-byte stores, marked
    // non-temporal (the kernel never reads C back: measured +4.6 % on
    // batched short-K products, whose C stores are a third of their time),
    // and with edges only rows < M and columns < N are touched.  With EPI the
    // bias of each column is added and the activation applied before the
    // store; the activation is chosen once, outside the unrolled stores.
    const int i = lane & 15, g = lane >> 4;
    const bool read_c = (p.beta != 0.f);
    const int row0 = m0 + wr * WM, col0 = n0 + wc * WN;
    float bcol[S::CB];   // bias of the column of acc[.][cb] (EPI)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb) {
        const int gn = col0 + (cb / 4) * 64 + 4 * i + cb % 4;
        bcol[cb] = (EPI && p.bias && (!GUARD || gn < p.N)) ? p.bias[gn] : 0.f;
    }
    auto store = [&](auto act_tag) {
        constexpr int ACT = decltype(act_tag)::value;   // -1: no epilogue
        auto finish = [&](float v, int cb) {
            if constexpr (ACT < 0)
                return v;
            else
                return activate_t<ACT>(v + bcol[cb]);
        };
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (rb < rlo || rb >= rhi) continue;
                const int gm = S::TRANS_A ? row0 + (rb / 4) * 64 + 16 * g + 4 * r + rb % 4
                                          : row0 + rb * 16 + 4 * g + r;
                if (GUARD && gm >= p.M) continue;
                float *crow = p.C + (long long)gm * p.ldc;
#pragma unroll
                for (int cg = 0; cg < S::CG; ++cg) {
                    const int gn = col0 + cg * 64 + 4 * i;
                    floatx4 v;
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = p.alpha * acc[rb][cg * 4 + c][r];
                    if (!GUARD || (cvec && gn + 3 < p.N)) {
                        floatx4 *dst = reinterpret_cast<floatx4 *>(crow + gn);
                        if (read_c) {
                            const floatx4 old = *dst;
#pragma unroll
                            for (int c = 0; c < 4; ++c) v[c] = fmaf(p.beta, old[c], v[c]);
                        }
#pragma unroll
                        for (int c = 0; c < 4; ++c) v[c] = finish(v[c], cg * 4 + c);
                        __builtin_nontemporal_store(v, dst);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            if (gn + c >= p.N) continue;
                            float out = v[c];
                            if (read_c) out = fmaf(p.beta, crow[gn + c], out);
                            crow[gn + c] = finish(out, cg * 4 + c);
                        }
                    }
                }
            }
    };
    if constexpr (EPI) {
        switch (p.act) {
        case SGEMM_ACT_RELU: store(std::integral_constant<int, SGEMM_ACT_RELU>{}); break;
        case SGEMM_ACT_SILU: store(std::integral_constant<int, SGEMM_ACT_SILU>{}); break;
        case SGEMM_ACT_GELU_ERF: store(std::integral_constant<int, SGEMM_ACT_GELU_ERF>{}); break;
        case SGEMM_ACT_GELU_TANH: store(std::integral_constant<int, SGEMM_ACT_GELU_TANH>{}); break;
        default: store(std::integral_constant<int, SGEMM_ACT_NONE>{}); break;
        }
    } else {
        store(std::integral_constant<int, -1>{});
    }
    };   // finish

    // the stream-K workspace: slot `slot` holds RB*CB floatx4 per thread,
    // laid out so that neighbouring threads touch neighbouring 16 bytes
    auto ws_at = [&](int slot, int j) {
        return reinterpret_cast<floatx4 *>(sk.ws) +
               ((long long)slot * (RB * S::CB) + j) * S::NT + tid;
    };
    auto coords = [&](int tile, int &m0, int &n0) {
        int tm, tn;
        tile_coords(tile, tiles_m, tiles_n, group_m, tm, tn);
        m0 = tm * BM;
        n0 = tn * BN;
    };

    if constexpr (MODE == 0) {
        int tm, tn;
        tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
        zero_acc();
        mainloop(tm * BM, tn * BN, 0, nk);
        finish(tm * BM, tn * BN, 0, RB);
    } else if constexpr (MODE == 1) {
        // whole tiles, numbered over the batch entries (the grid has one row):
        // each XCD takes a contiguous range of them, so the panels its tiles
        // share stay in its L2
        int m0, n0;
        const int per_entry = tiles_m * tiles_n;
        const float *A0 = p.A, *B0 = p.B;
        float *C0 = p.C;
        for (int tile = blockIdx.x; tile < sk.dp_tiles; tile += sk.groups) {
            const int lt = xcd_remap(tile, sk.dp_tiles);
            const int b = lt / per_entry;
            p.A = A0 + b * p.stride_a;
            p.B = B0 + b * p.stride_b;
            p.C = C0 + b * p.stride_c;
            coords(lt - b * per_entry, m0, n0);
            zero_acc();
            mainloop(m0, n0, 0, nk);
            finish(m0, n0, 0, RB);
            __syncthreads();   // LDS free for the next tile's loads
        }
        p.A = A0;
        p.B = B0;
        p.C = C0;
        // run v of the split tiles: consecutive runs (and so neighbouring
        // tiles, which share panels of A and B) on one XCD
        const int v = xcd_remap(blockIdx.x, sk.groups);
        const long long total = (long long)sk.sk_tiles * sk.iters;
        long long it = (long long)v * sk.per_wg;
        const long long end = it + sk.per_wg < total ? it + sk.per_wg : total;
        while (it < end) {
            const int tl = (int)(it / sk.iters);
            const int k0 = (int)(it - (long long)tl * sk.iters);
            const int k1 = (long long)sk.iters - k0 < end - it ? sk.iters : k0 + (int)(end - it);
            coords(sk.dp_tiles + tl, m0, n0);
            zero_acc();
            mainloop(m0, n0, k0, k1);
            if (k0 == 0 && k1 == sk.iters) {
                finish(m0, n0, 0, RB);
            } else {
                const int slot = 2 * v + (it == (long long)v * sk.per_wg ? 0 : 1);
#pragma unroll
                for (int x = 0; x < RB; ++x)
#pragma unroll
                    for (int y = 0; y < S::CB; ++y) *ws_at(slot, x * S::CB + y) = acc[x][y];
            }
            it += k1 - k0;
            __syncthreads();   // LDS free for the next piece's loads
        }
    } else {
        // fixup: workgroup (tl, z) adds row block z of every wave over the
        // pieces of stream-K tile tl and stores it; tiles of one piece are done
        const int tl = blockIdx.x, z = blockIdx.y;
        const int pieces = sk_pieces(sk, tl);
        if (pieces == 1) return;
        zero_acc();
        for (int q = 0; q < pieces; ++q) {
            const int slot = sk_slot(sk, tl, q);
#pragma unroll
            for (int x = 0; x < RB; ++x) {
                if (x != z) continue;
#pragma unroll
                for (int y = 0; y < S::CB; ++y) {
                    const floatx4 v = *ws_at(slot, x * S::CB + y);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[x][y][e] += v[e];
                }
            }
        }
        int m0, n0;
        coords(sk.dp_tiles + tl, m0, n0);
        finish(m0, n0, z, z + 1);
    }
}

template <int BM, int BN, int BK, int WM, int WN, int NBUF, int KG, bool TB, bool TA, int AV,
          int BV, bool GUARD, bool EPI = false, int IN = 0>
hipError_t launch_one(const Problem &p, int group_m, bool cvec, hipStream_t stream) {
    using S = DirectShape<BM, BN, BK, WM, WN, NBUF, AV, BV, KG, TB, TA, EPI, IN>;
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const long long tiles = (long long)tiles_m * tiles_n;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (group_m <= 0) group_m = 4;
    hipLaunchKernelGGL(
        (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, AV, BV, GUARD, EPI, IN>),
        dim3((unsigned)tiles, p.batch), dim3(S::NT), 0, stream, p, tiles_m, tiles_n, group_m,
        (int)cvec, StreamK{});
    return hipGetLastError();
}

// Picks the kernel instance for the operands: the whole-tile instance when
// the problem is made of whole tiles with 16-byte rows everywhere, else (for
// tiles compiled with EDGES) a guarded instance with dwordx4 loads for each
// operand whose rows allow them (16-byte aligned rows, and the length along
// the row -- K, or N for untransposed B -- a multiple of 4, so that a 16-byte
// chunk is entirely inside or outside the matrix).  A k-contiguous operand
// (A untransposed, B transposed) whose rows do not allow them takes dwordx4
// loads from its 4-byte aligned rows with the k-tail stage split into dword
// loads (load width 5); the others take dword loads.  Transposed B is served
// by the EDGES tiles only.  VEC = false (4-byte I/O asked for) uses dword
// loads and scalar stores.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int KG, bool TB, bool TA, bool EDGES,
          bool VEC>
hipError_t launch_for(const Problem &p, int group_m, hipStream_t stream) {
    const bool whole = p.M % BM == 0 && p.N % BN == 0 && p.K % BK == 0;
    const bool av = VEC && rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) &&
                    (TA ? p.M : p.K) % 4 == 0;
    const bool bv = VEC && rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4) &&
                    (TB ? p.K : p.N) % 4 == 0;
    const bool cv = VEC && rows_aligned(p.C, p.ldc, p.stride_c, p.batch, 4);
    if constexpr (!TB && !TA) {
        if (whole && av && bv && cv)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, 4, 4, false>(p, group_m, true,
                                                                                stream);
    }
    if constexpr (EDGES) {
        constexpr int AS = TA ? 1 : 5, BS = TB ? 5 : 1;   // widths for rows without 16-byte loads
        if (!VEC)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, 1, 1, true>(p, group_m, cv,
                                                                               stream);
        if (av && bv)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, 4, 4, true>(p, group_m, cv,
                                                                               stream);
        if (av)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, 4, BS, true>(p, group_m, cv,
                                                                                stream);
        if (bv)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, AS, 4, true>(p, group_m, cv,
                                                                                stream);
        return launch_one<BM, BN, BK, WM, WN, NBUF, KG, TB, TA, AS, BS, true>(p, group_m, cv,
                                                                             stream);
    }
    return hipErrorInvalidValue;
}

// TA: the tile table this entry belongs to serves A stored transposed (and
// only that); B may be transposed or not on tiles with EDGES.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int KG, bool TA, bool EDGES, bool VEC>
hipError_t launch_direct(const Problem &p, int group_m, hipStream_t stream) {
    if ((p.trans_a != 0) != TA) return hipErrorInvalidValue;
    if (!direct_applies(p, BM, BN, BK, EDGES)) return hipErrorInvalidValue;
    if (p.trans_b) {
        if constexpr (EDGES)
            return launch_for<BM, BN, BK, WM, WN, NBUF, KG, true, TA, EDGES, VEC>(p, group_m,
                                                                                 stream);
        return hipErrorInvalidValue;
    }
    return launch_for<BM, BN, BK, WM, WN, NBUF, KG, false, TA, EDGES, VEC>(p, group_m, stream);
}

// The fused-epilogue launcher: bias and activation applied in the kernel's
// own epilogue, for operands that take dwordx4 loads of A and B (the
// instances compiled with EPI); hipErrorNotSupported otherwise.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int KG, bool TA, bool EDGES>
hipError_t launch_direct_epi(const Problem &p, int group_m, hipStream_t stream) {
    if ((p.trans_a != 0) != TA) return hipErrorInvalidValue;
    if (!direct_applies(p, BM, BN, BK, EDGES)) return hipErrorInvalidValue;
    const bool tb = p.trans_b != 0;
    const bool av = rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) && (TA ? p.M : p.K) % 4 == 0;
    const bool bv = rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4) && (tb ? p.K : p.N) % 4 == 0;
    const bool cv = rows_aligned(p.C, p.ldc, p.stride_c, p.batch, 4);
    if (!av || !bv) return hipErrorNotSupported;
    const bool whole = p.M % BM == 0 && p.N % BN == 0 && p.K % BK == 0;
    if constexpr (!TA) {
        if (!tb && whole && cv)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, false, false, 4, 4, false, true>(
                p, group_m, true, stream);
    }
    if constexpr (EDGES) {
        if (tb)
            return launch_one<BM, BN, BK, WM, WN, NBUF, KG, true, TA, 4, 4, true, true>(p, group_m,
                                                                                      cv, stream);
        return launch_one<BM, BN, BK, WM, WN, NBUF, KG, false, TA, 4, 4, true, true>(p, group_m,
                                                                                   cv, stream);
    }
    return hipErrorNotSupported;
}

// The launcher for 16-bit inputs (IN = 1 or 2).  `pw` is the problem in
// 32-bit words along k (K, lda, ldb halved; A untransposed, B transposed, so
// each word holds two adjacent k values); it takes dwordx4 loads when both
// operands' word rows allow them, and otherwise split-tail loads (width 5,
// as launch_for) from the 4-byte aligned word rows.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, int KG, int IN>
hipError_t launch_direct16(const Problem &pw, int group_m, hipStream_t stream) {
    if (pw.trans_a || !pw.trans_b) return hipErrorInvalidValue;
    if (!direct_applies(pw, BM, BN, BK, true)) return hipErrorInvalidValue;
    const bool av = rows_aligned(pw.A, pw.lda, pw.stride_a, pw.batch, 4) && pw.K % 4 == 0;
    const bool bv = rows_aligned(pw.B, pw.ldb, pw.stride_b, pw.batch, 4) && pw.K % 4 == 0;
    const bool cv = rows_aligned(pw.C, pw.ldc, pw.stride_c, pw.batch, 4);
    if (av && bv)
        return launch_one<BM, BN, BK, WM, WN, NBUF, KG, true, false, 4, 4, true, false, IN>(
            pw, group_m, cv, stream);
    // otherwise dwordx4 loads from 4-byte aligned word rows, dword loads on the k tail
    return launch_one<BM, BN, BK, WM, WN, NBUF, KG, true, false, 5, 5, true, false, IN>(
        pw, group_m, cv, stream);
}

// Workgroups of a stream-K launch: one per CU (the tiles that offer stream-K
// run one 8-wave workgroup per CU).
constexpr int kStreamKGroups = 256;

// Stream-K launch of a tile with one k-group (dwordx4 loads of A and B, the
// guarded instance): the plan, the workspace (workspace_acquire), the runs
// and the fixup.  The last full wave of tiles and the remainder are split
// (the tiles before them run whole), so every workgroup gets the same number
// of k-iterations.  A batch (at most kMaxBatchPerLaunch entries) runs the
// same persistent workgroups over the whole tiles of all its entries, with
// no split.  hipErrorNotSupported when the operands do not take dwordx4
// loads.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, bool TA>
hipError_t launch_streamk(const Problem &p, int group_m, hipStream_t stream) {
    if ((p.trans_a != 0) != TA) return hipErrorInvalidValue;
    if (!direct_applies(p, BM, BN, BK, true)) return hipErrorInvalidValue;
    const bool tb = p.trans_b != 0;
    const bool av = rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) && (TA ? p.M : p.K) % 4 == 0;
    const bool bv = rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4) && (tb ? p.K : p.N) % 4 == 0;
    const bool cv = rows_aligned(p.C, p.ldc, p.stride_c, p.batch, 4);
    if (!av || !bv) return hipErrorNotSupported;
    using S = DirectShape<BM, BN, BK, WM, WN, NBUF, 4, 4, 1, false, TA>;
    const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const long long tiles = (long long)tiles_m * tiles_n;
    const int G = kStreamKGroups;
    if (tiles * p.batch > 0x7fffffffLL / 16) return hipErrorInvalidConfiguration;
    if (group_m <= 0) group_m = 4;
    StreamK sk;
    if (p.batch > 1) {
        // a batch: persistent workgroups over the whole tiles of every entry
        // (a tile's stores drain while the workgroup loads its next tile); no
        // split, no workspace
        sk.dp_tiles = (int)(tiles * p.batch);
        sk.groups = sk.dp_tiles < G ? sk.dp_tiles : G;
        sk.iters = (p.K + BK - 1) / BK;
        sk.per_wg = 1;
        Problem q = p;
        q.batch = 1;   // the grid has one row; the kernel walks the entries
        if (tb)
            hipLaunchKernelGGL(
                (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, 1, true, TA, 4, 4, true, false, 0, 1>),
                dim3(sk.groups), dim3(S::NT), 0, stream, q, tiles_m, tiles_n, group_m, (int)cv, sk);
        else
            hipLaunchKernelGGL(
                (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, 1, false, TA, 4, 4, true, false, 0, 1>),
                dim3(sk.groups), dim3(S::NT), 0, stream, q, tiles_m, tiles_n, group_m, (int)cv, sk);
        return hipGetLastError();
    }
    sk.groups = G;
    sk.dp_tiles = tiles >= G ? (int)((tiles / G - 1) * G) : 0;
    sk.sk_tiles = (int)(tiles - sk.dp_tiles);
    sk.iters = (p.K + BK - 1) / BK;
    const long long sk_iters = (long long)sk.sk_tiles * sk.iters;
    if (sk_iters / G > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    sk.per_wg = (int)((sk_iters + G - 1) / G);
    const size_t bytes = (size_t)2 * G * (S::RB * S::CB) * S::NT * 16;   // two slots a run
    Workspace w;
    hipError_t e = workspace_acquire(bytes, stream, p, w);
    if (e != hipSuccess) return e;
    sk.ws = static_cast<float *>(w.ptr);
    if (tb)
        hipLaunchKernelGGL(
            (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, 1, true, TA, 4, 4, true, false, 0, 1>),
            dim3(G), dim3(S::NT), 0, stream, p, tiles_m, tiles_n, group_m, (int)cv, sk);
    else
        hipLaunchKernelGGL(
            (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, 1, false, TA, 4, 4, true, false, 0, 1>),
            dim3(G), dim3(S::NT), 0, stream, p, tiles_m, tiles_n, group_m, (int)cv, sk);
    e = hipGetLastError();
    if (e == hipSuccess) {
        if (tb)
            hipLaunchKernelGGL(
                (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, 1, true, TA, 4, 4, true, false, 0, 2>),
                dim3(sk.sk_tiles, S::RB), dim3(S::NT), 0, stream, p, tiles_m, tiles_n, group_m, (int)cv,
                sk);
        else
            hipLaunchKernelGGL(
                (mfma_direct_kernel<BM, BN, BK, WM, WN, NBUF, 1, false, TA, 4, 4, true, false, 0,
                                    2>),
                dim3(sk.sk_tiles, S::RB), dim3(S::NT), 0, stream, p, tiles_m, tiles_n, group_m, (int)cv,
                sk);
        e = hipGetLastError();
    }
    const hipError_t f = workspace_release(w, stream);
    return e != hipSuccess ? e : f;
}

// The stream-K launcher of a tile table entry, or none: offered by the
// 256-row tiles with edges and one k-group.
template <int BM, int BN, int BK, int WM, int WN, int NBUF, bool EDGES, int KG, bool TA>
constexpr LaunchFn streamk_launcher() {
    if constexpr (EDGES && KG == 1 && BM == 256)
        return &launch_streamk<BM, BN, BK, WM, WN, NBUF, TA>;
    else
        return nullptr;
}

// Tile-table entry of a direct-load tile.  Tiles without EDGES serve whole
// tiles of untransposed operands only; tiles with EDGES also serve transposed
// B.  TA tiles serve transposed A (and only that), with B either way.  The
// fused-epilogue launchers are compiled in their own translation units and
// joined to the entries by the dispatcher (fused_launchers).
template <int BM, int BN, int BK, int WM, int WN, int NBUF, bool EDGES, int KG = 1,
          bool TA = false>
constexpr TileEntry direct_entry(int eff_pct) {
    static_assert(EDGES || !TA, "transposed-A tiles are compiled with edges");
    using S = DirectShape<BM, BN, BK, WM, WN, NBUF, 4, 4, KG, false, TA>;
    return TileEntry{{BM, BN, BK, WM, WN, 0, 0, S::NT, S::LDS_BYTES, NBUF,
                      SGEMM_TILE_DIRECT | (EDGES ? SGEMM_TILE_TRANS_B : SGEMM_TILE_WHOLE) |
                          (TA ? SGEMM_TILE_TRANS_A : 0)},
                     &launch_direct<BM, BN, BK, WM, WN, NBUF, KG, TA, EDGES, true>,
                     EDGES ? &launch_direct<BM, BN, BK, WM, WN, NBUF, KG, TA, EDGES, false>
                           : nullptr,
                     eff_pct};
}

}  // namespace
}  // namespace sg
