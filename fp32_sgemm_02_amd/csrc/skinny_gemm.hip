// skinny_gemm.hip -- SGEMM shapes with few rows (M <= 16) or few columns
// (N <= 16) of C.  They do O(1) flops per byte of the large operand, far below
// the ridge point of the roofline ("The GEMM Scrapbook", roofline paragraph:
// peak flops over memory bandwidth), so they are bound by HBM: the kernels
// stream the large operand exactly once, with every wave keeping several
// 16-byte loads per lane in flight.
//
// Every load is a buffer load whose offset is computed without branches: a
// lane whose element lies outside the matrix (or outside its K slice) gets an
// offset past the buffer's range, and the hardware returns zeros without
// touching memory ("The 1% kernel" section 6: idle threads past the matrix).
// Per-lane branches around the loads would make the compiler wait for every
// load in flight at each branch join, one load at a time.
//
// Few rows (kind 0): C (M x N) = A (M x K) * B (K x N), B streamed.  The M <= 16
// rows of A are the A operand of v_mfma_f32_16x16x4_f32 (rows >= M read as
// zero).  A wave owns 64*Q columns of C; lane l (i = l % 16, g = l / 16)
// supplies, in MFMA step s of a 16-row k-chunk, k = 4g + s, and loads four
// consecutive B values of row k at columns 64q + 4i .. +3 for each q < Q:
// the 16 lanes of a row group read 256 contiguous bytes per load, 256*Q per
// row in all ("a CUDA matmul" section 04: neighbouring lanes on neighbouring
// addresses).  Column 64q + 4i + c feeds MFMA column block 4q + c, whose
// result register r is C[4g + r][64q + 4i + c].  The WK waves of a
// workgroup share its columns and take turns over the 16-row k-chunks; their
// sums meet in LDS in a fixed order.
//
// Schedule.  A workgroup owns one strip of 64*Q columns and one slice of K.
// With S > 1 slices the slices' partial sums go to a workspace and the last
// workgroup of a strip to arrive (an atomic counter per strip) adds them in
// slice order and writes C: the result does not depend on which workgroup
// finishes last, and one launch does the whole product.  HBM is saturated
// only when every CU streams, so skinny products whose strips are fewer than
// the CUs are split; the small tiles fit several workgroups per CU, so that
// one workgroup's closing reduction overlaps the others' loads.
//
// Few columns (kind 1): each wave owns R rows of A and walks them with 16-byte
// loads along k, multiplying by the N <= NB columns of B (small, cache
// resident; one load of B serves the R rows), then reduces its 64 lanes.
//
// Transposed storage.  B stored N x K (a linear layer's weight, C = X W^T):
// in kind 0 a lane loads the four k values 4g .. 4g+3 of a column from that
// column's row of B^T (one 16-byte load per column, the MFMA operand of all
// four steps); in kind 1 the N <= NB rows of B^T are read 16 bytes at a time
// like A's rows.  A stored K x M is served by kind 0 only (its <= 16 columns
// are read four bytes at a time; A is small).
#include <cstdint>

#include "gemm_internal.hpp"

namespace sg {
namespace {

// A buffer offset past every resource's range (records are below 2^31).
constexpr int kOff = (int)0x80000000u;

// Raw buffer resource over [base, base + bytes), capped at 2^31 - 1 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base, long long bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n, 0x00020000);
}

// 16-byte and 4-byte buffer loads; NT: non-temporal (data streamed once).
template <bool NT>
__device__ __forceinline__ floatx4 ld4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(floatx4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0));
}
__device__ __forceinline__ float ld1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// The finished value of one cell: alpha * sum (+ beta * C) (+ bias, act).
__device__ __forceinline__ void store_cell(const Problem &p, float *dst, int col, float sum) {
    float out = p.alpha * sum;
    if (p.beta != 0.f) out = fmaf(p.beta, *dst, out);
    if (p.has_epilogue()) out = activate(p.act, p.bias ? out + p.bias[col] : out);
    *dst = out;
}

// ---------------------------------------------------------------- kind 0 ----
// The split of a few-rows launch: workgroup w owns strip w % strips (columns
// [strip * width, min(N, (strip + 1) * width))) and K slice w / strips, rows
// [slice * kslice, min(K, (slice + 1) * kslice)).
struct RowsGrid {
    int strips;        // column strips
    int width;         // columns per strip: a multiple of 4, at most 64*Q
    int slices;        // K slices (1: no split, no workspace)
    int kslice;        // rows of K per slice, a multiple of 16
    float *part;       // slices x M x N partial sums (row-major, leading dimension N)
    unsigned *count;   // one arrival counter per strip, zero between launches
};

template <int Q, int WK, int U>
struct RowsShape {
    static constexpr int NT = 64 * WK;
    static constexpr int COLS = 64 * Q;
    static constexpr int ACC = 4 * Q;                    // floatx4 accumulators per lane
    static constexpr int LDS_BYTES = WK * ACC * 64 * 16;
    static_assert(LDS_BYTES <= 64 * 1024, "wave sums of a workgroup fit 64 KB of LDS");
};

// One round of a wave's loads: U consecutive 16-row k-chunks.
// B untransposed: b[u][s][q] = B(k0 + s, 64q + 4i + 0..3);
// B transposed:   b[u][c][q] = B(k0 + 0..3, 64q + 4i + c);
// a[u] = A(row i, k0 + 0..3); k0 = 16 * chunk + 4g.
template <int Q, int U>
struct RowsRound {
    floatx4 b[U][4][Q];
    floatx4 a[U];
};

// VA / VB: 16-byte loads of A / B (rows 16-byte aligned, the stored row length
// a multiple of 4, so a group of four never straddles the edge).  kr0 is the
// first row of K of the round's U consecutive chunks (uniform over the
// wave): for B stored transposed, the four lanes of a column read 64
// contiguous bytes per chunk, so a round reads 64*U per column.  Each
// chunk (and, for B^T, each 64-column group) gets a resource of its own that
// starts at its first row (column), so the per-lane offsets stay below 2^31
// for any K: under 16 * ldb floats for B, 64 * ldb for B^T, 16 * lda for A.
template <int Q, int WK, int U, bool VA, bool VB, bool TA, bool TB>
__device__ __forceinline__ void rows_load(const Problem &p, int ke, int n0, int ncols, int kr0,
                                          int i, int g, RowsRound<Q, U> &r) {
    const int ldb = (int)p.ldb, lda = (int)p.lda;
    const int kk = 4 * g;   // this lane's first row of a chunk
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int kr = kr0 + 16 * u;   // the chunk's first row
        const int krem = ke - kr;            // rows of the slice from kr on
        if constexpr (TB) {
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const __amdgpu_buffer_rsrc_t rb =
                    make_rsrc(p.B + (long long)(n0 + 64 * q) * p.ldb + kr,
                              4 * ((long long)(ncols - 64 * q - 1) * p.ldb + krem));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int col = 4 * i + c;   // within the 64-column group
                    const bool ok = 64 * q + col < ncols;
                    if constexpr (VB) {
                        r.b[u][c][q] = ld4<false>(rb, (ok && kk < krem) ? (col * ldb + kk) * 4 : kOff);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            r.b[u][c][q][e] =
                                ld1(rb, (ok && kk + e < krem) ? (col * ldb + kk + e) * 4 : kOff);
                    }
                }
            }
        } else {
            // rows of the chunk past the slice fall outside the resource (its
            // records end at row min(krem, 16)), so the 16-byte loads' offsets
            // depend on the lane only and stay in registers across rounds
            const int rows = krem < 16 ? (krem > 0 ? krem : 0) : 16;
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(p.B + (long long)kr * p.ldb + n0, 4LL * rows * p.ldb);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool rok = kk + s < krem;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int col = 64 * q + 4 * i;
                    if constexpr (VB) {
                        r.b[u][s][q] = ld4<true>(rb, col < ncols ? ((kk + s) * ldb + col) * 4 : kOff);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            r.b[u][s][q][c] = ld1(
                                rb, (rok && col + c < ncols) ? ((kk + s) * ldb + col + c) * 4 : kOff);
                    }
                }
            }
        }
        const bool mok = i < p.M;
        if constexpr (TA) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(
                p.A + (long long)kr * p.lda, 4 * ((long long)(krem - 1) * p.lda + p.M));
#pragma unroll
            for (int e = 0; e < 4; ++e)
                r.a[u][e] = ld1(ra, (mok && kk + e < krem) ? ((kk + e) * lda + i) * 4 : kOff);
        } else {
            const __amdgpu_buffer_rsrc_t ra =
                make_rsrc(p.A + kr, 4 * ((long long)(p.M - 1) * p.lda + krem));
            if constexpr (VA) {
                r.a[u] = ld4<false>(ra, (mok && kk < krem) ? (i * lda + kk) * 4 : kOff);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r.a[u][e] = ld1(ra, (mok && kk + e < krem) ? (i * lda + kk + e) * 4 : kOff);
            }
        }
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// IN = 1 / 2: 16-bit inputs in word form (see the 16-bit family): a lane's
// four k-words of A and of a column are the 8 k values of one
// v_mfma_f32_16x16x32 (bfloat16 / float16).
template <int Q, int U, bool TB, int IN>
__device__ __forceinline__ void rows_mfma(const RowsRound<Q, U> &r, floatx4 (&acc)[4 * Q]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (IN != 0) {
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if constexpr (IN == 1)
                        acc[4 * q + c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, r.a[u]),
                            __builtin_bit_cast(bf16x8, r.b[u][c][q]), acc[4 * q + c], 0, 0, 0);
                    else
                        acc[4 * q + c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            __builtin_bit_cast(f16x8, r.a[u]),
                            __builtin_bit_cast(f16x8, r.b[u][c][q]), acc[4 * q + c], 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float b = TB ? r.b[u][c][q][s] : r.b[u][s][q][c];
                        acc[4 * q + c] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            r.a[u][s], b, acc[4 * q + c], 0, 0, 0);
                    }
        }
    }
}

// Cell (m, col) of a strip from the waves' sums in LDS, added in wave
// order: register m % 4 of accumulator 4 (col / 64) + col % 4 of lane
// 16 (m / 4) + (col % 64) / 4.
template <int Q, int WK>
__device__ __forceinline__ float wave_sum(const floatx4 (&red)[WK][4 * Q][64], int m, int col) {
    const int a = 4 * (col >> 6) + (col & 3), l = 16 * (m >> 2) + ((col & 63) >> 2);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WK; ++w) sum += red[w][a][l][m & 3];
    return sum;
}

// The end of a few-rows workgroup: the waves' sums meet in LDS (red), then
// the workgroup stores its cells of C (one slice), or its partial sums, and
// the last workgroup of the strip to arrive adds the slices in order.
template <int Q, int WK>
__device__ __forceinline__ void rows_finish(const Problem &p, const RowsGrid &grid,
                                            floatx4 (&red)[WK][4 * Q][64], int &last,
                                            const floatx4 (&acc)[4 * Q], int tid, int strip,
                                            int slice, int n0, int ncols) {
    using S = RowsShape<Q, WK, 1>;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int a = 0; a < 4 * Q; ++a) red[wave][a][lane] = acc[a];
    __syncthreads();
    const int cells = p.M * S::COLS;
    if (grid.slices == 1) {
        for (int f = tid; f < cells; f += S::NT) {
            const int m = f / S::COLS, col = f % S::COLS;
            if (col < ncols)
                store_cell(p, p.C + (long long)m * p.ldc + n0 + col, n0 + col,
                           wave_sum<Q, WK>(red, m, col));
        }
        return;
    }
    float *part = grid.part + (long long)slice * p.M * p.N;
    for (int f = tid; f < cells; f += S::NT) {
        const int m = f / S::COLS, col = f % S::COLS;
        if (col < ncols)
            __hip_atomic_store(part + (long long)m * p.N + n0 + col, wave_sum<Q, WK>(red, m, col),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial sums have completed
    __syncthreads();
    if (tid == 0)
        last = __hip_atomic_fetch_add(grid.count + strip, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(grid.slices - 1);
    __syncthreads();
    if (!last) return;
    const long long step = (long long)p.M * p.N;
    for (int f = tid; f < cells; f += S::NT) {
        const int m = f / S::COLS, col = f % S::COLS;
        if (col >= ncols) continue;
        const float *src = grid.part + (long long)m * p.N + n0 + col;
        // slice order kept; sixteen slices' loads in flight at a time
        float sum = 0.f;
        for (int z = 0; z < grid.slices; z += 16) {
            float v[16];
#pragma unroll
            for (int x = 0; x < 16; ++x)
                v[x] = z + x < grid.slices
                           ? __hip_atomic_load(src + (z + x) * step, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0.f;
#pragma unroll
            for (int x = 0; x < 16; ++x)
                if (z + x < grid.slices) sum += v[x];
        }
        store_cell(p, p.C + (long long)m * p.ldc + n0 + col, n0 + col, sum);
    }
    if (tid == 0)   // ready for the next launch on the stream
        __hip_atomic_store(grid.count + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Each wave walks its chunks of a strip segment in rounds of U with two
// register sets: the loads of round r + 1 are issued before the MFMAs of
// round r, so a round's memory latency overlaps the previous round's
// arithmetic (chunks past the segment read as zero and touch no memory).
//
// Partial sums are written and read as device-coherent (agent-scope)
// accesses, which bypass the per-XCD caches that are not coherent with each
// other; every wave waits for its stores to complete before the workgroup
// counts its arrival, so the workgroup that counts last finds every partial
// sum in memory.  (A release fence would also write back each XCD's whole L2,
// once per wave: measured to cost more than the split saves.)
template <int Q, int WK, int U, bool VA, bool VB, bool TA, bool TB, int IN = 0>
__global__ void __launch_bounds__(64 * WK) rows_kernel(Problem p, RowsGrid grid) {
    static_assert(IN == 0 || (TB && !TA), "16-bit inputs: B transposed (word form)");
    using S = RowsShape<Q, WK, U>;
    __shared__ floatx4 red[WK][S::ACC][64];
    __shared__ int last;
    select_batch(p);
    // the wave index is uniform over the wave: in a scalar register, so the
    // buffer resources built from it are too
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int strip = blockIdx.x % grid.strips, slice = blockIdx.x / grid.strips;
    const int n0 = strip * grid.width, ncols = min(grid.width, p.N - n0);
    const int kb = slice * grid.kslice, ke = min(p.K, kb + grid.kslice);
    const int c1 = (ke - kb + 15) / 16;   // chunks of the slice

    floatx4 acc[S::ACC];
#pragma unroll
    for (int a = 0; a < S::ACC; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
    // wave w takes the groups of U consecutive chunks w, w + WK, ...
    const int groups = (c1 + U - 1) / U;
    RowsRound<Q, U> r0, r1;
    rows_load<Q, WK, U, VA, VB, TA, TB>(p, ke, n0, ncols, kb + 16 * U * wave, i, g, r0);
    for (int j = wave; j < groups; j += 2 * WK) {
        rows_load<Q, WK, U, VA, VB, TA, TB>(p, ke, n0, ncols, kb + 16 * U * (j + WK), i, g, r1);
        pipeline_fence();
        rows_mfma<Q, U, TB, IN>(r0, acc);
        if (j + WK >= groups) break;
        rows_load<Q, WK, U, VA, VB, TA, TB>(p, ke, n0, ncols, kb + 16 * U * (j + 2 * WK), i, g, r0);
        pipeline_fence();
        rows_mfma<Q, U, TB, IN>(r1, acc);
    }
    rows_finish<Q, WK>(p, grid, red, last, acc, tid, strip, slice, n0, ncols);
}

// B stored transposed, staged through LDS (64 columns, four waves, rounds of
// four 16-row k-chunks).  Loading B^T straight into the MFMA layout gives
// each column's row of B^T to four lanes, 64 contiguous bytes per row and
// load; here each wave copies its round (64 rows of B^T and the <= 16 rows of
// A, 64 k each) into LDS buffers of its own with direct global-to-LDS loads in
// which 16 lanes read 256 contiguous bytes of one row, then reads its MFMA
// operands from LDS.  Row r of a B buffer holds the 16 four-float pieces of
// its 64 k in slots piece ^ (r >> 2), row r of an A buffer in slots
// piece ^ r, so that the 16 lanes of an operand read (B rows 4i + c, A rows
// i, one piece each) hit 16 different slots: no bank conflicts.  Two buffers
// per wave: round j + 1 is in flight while round j is consumed.  Every load
// of the loop goes to LDS, so the only waits are the wave's own counts of
// its loads (no barrier in the loop); a buffer is refilled only after the
// MFMAs that used its previous contents, which waited for their LDS reads.
constexpr int kStagedFloats = 64 * 64 + 16 * 64;   // one round: B^T, then A

// Issue round kr .. kr + 63 of the slice ending at ke into `buf`.
__device__ __forceinline__ void staged_issue(const Problem &p, float *buf, int n0, int ncols,
                                             int kr, int ke, int lane) {
    const int ldb = (int)p.ldb, lda = (int)p.lda, krem = ke - kr;
    const int rsub = lane >> 4, slot = lane & 15;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.B + (long long)n0 * p.ldb + kr, 4 * ((long long)(ncols - 1) * p.ldb + krem));
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int r = 4 * q + rsub, k = 4 * (slot ^ q);
        const int off = (r < ncols && k < krem) ? (r * ldb + k) * 4 : kOff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void *)(buf + 256 * q), 16, off, 0, 0, 0);
    }
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A + kr, 4 * ((long long)(p.M - 1) * p.lda + krem));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = 4 * q + rsub, k = 4 * (slot ^ r);
        const int off = (r < p.M && k < krem) ? (r * lda + k) * 4 : kOff;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void *)(buf + 64 * 64 + 256 * q), 16, off, 0, 0,
            0);
    }
}

// The MFMAs of the round in `buf`, once its loads have landed (the 20 loads
// of the next round may still be in flight).  IN: input format as in
// rows_mfma (16-bit inputs in word form: k counts 32-bit words).
template <int IN>
__device__ __forceinline__ void staged_consume(const float *buf, int lane, floatx4 (&acc)[4]) {
    __builtin_amdgcn_s_waitcnt((20 & 15) | ((20 >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    const int i = lane & 15, g = lane >> 4;
    RowsRound<1, 4> r;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        r.a[u] = *reinterpret_cast<const floatx4 *>(buf + 64 * 64 + i * 64 + 4 * ((4 * u + g) ^ i));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int row = 4 * i + c, slot = (4 * u + g) ^ i;
            r.b[u][c][0] = *reinterpret_cast<const floatx4 *>(buf + row * 64 + 4 * slot);
        }
    }
    rows_mfma<1, 4, true, IN>(r, acc);
}

template <int WK, int IN>
__global__ void __launch_bounds__(64 * WK) rows_tb_staged_kernel(Problem p, RowsGrid grid) {
    using S = RowsShape<1, WK, 4>;
    // two buffers per wave, as separate arrays so that the compiler can tell a
    // read of one from the direct loads into the other; the waves' sums (and
    // the arrival flag) reuse the first array after the loop
    __shared__ __attribute__((aligned(1024))) float stage0[WK][kStagedFloats];
    __shared__ __attribute__((aligned(1024))) float stage1[WK][kStagedFloats];
    static_assert(sizeof(floatx4) * WK * S::ACC * 64 + 16 <= sizeof(float) * WK * kStagedFloats,
                  "the waves' sums fit the first buffer array");
    select_batch(p);
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int strip = blockIdx.x % grid.strips, slice = blockIdx.x / grid.strips;
    const int n0 = strip * grid.width, ncols = min(grid.width, p.N - n0);
    const int kb = slice * grid.kslice, ke = min(p.K, kb + grid.kslice);
    const int c1 = (ke - kb + 15) / 16;

    floatx4 acc[S::ACC];
#pragma unroll
    for (int a = 0; a < S::ACC; ++a) acc[a] = floatx4{0.f, 0.f, 0.f, 0.f};
    float *buf0 = stage0[wave], *buf1 = stage1[wave];
    const int groups = (c1 + 3) / 4;   // rounds of 64 k; wave w takes w, w + WK, ...
    staged_issue(p, buf0, n0, ncols, kb + 64 * wave, ke, lane);
    for (int j = wave; j < groups; j += 2 * WK) {
        staged_issue(p, buf1, n0, ncols, kb + 64 * (j + WK), ke, lane);
        pipeline_fence();
        staged_consume<IN>(buf0, lane, acc);
        if (j + WK >= groups) break;
        staged_issue(p, buf0, n0, ncols, kb + 64 * (j + 2 * WK), ke, lane);
        pipeline_fence();
        staged_consume<IN>(buf1, lane, acc);
    }
    // every wave's last (zero-filling) loads have landed before the buffers
    // are reused for the sums
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    auto &red = *reinterpret_cast<floatx4 (*)[WK][S::ACC][64]>(&stage0[0][0]);
    int &last = *reinterpret_cast<int *>(&red[WK - 1][S::ACC - 1][63] + 1);
    rows_finish<1, WK>(p, grid, red, last, acc, tid, strip, slice, n0, ncols);
}

// Counters of the workspace: one per strip, so a split launch has at most
// this many strips.
constexpr int kMaxSplitStrips = kWorkspaceCounters;

// K slices of a few-rows launch: `want` when given (at most 64, and one
// 16-row chunk per wave and slice), else the library's choice for single
// products whose strips are fewer than the CUs: as many slices as keep the
// grid within about one workgroup per CU (measured best over M = 1..16,
// N = 256..14336, K = 3001..16384: HBM is saturated only while every CU
// streams, and a second round of workgroups costs more than it balances),
// with every wave still running two rounds of loads or more where that leaves
// 128 workgroups or more (1 x 256 x 16384: 32 slices 8.7 us, 64 slices 10.6;
// 1 x 512 x 8192: 16 slices 8.1 us, 32 slices 9.2), else one round at least
// (the one-row edge strip of 4097 x 1000 x 3001: 11 slices 7.8 us, 5 slices
// 9.2), and the partial sums (written and read once) under ~3 % of B's bytes.
template <int Q, int WK, int U>
int rows_slices(const Problem &p, int want) {
    using S = RowsShape<Q, WK, U>;
    const long long strips = (p.N + S::COLS - 1) / S::COLS;
    if (p.batch != 1 || p.K == 0 || strips > kMaxSplitStrips) return 1;
    const long long chunks = (p.K + 15) / 16;
    long long s;
    if (want > 0) {
        s = want < 64 ? want : 64;
        if (s > (chunks + WK - 1) / WK) s = (chunks + WK - 1) / WK;
    } else {
        s = 256 / strips;
        const long long two = chunks / (2LL * WK * U), one = chunks / ((long long)WK * U);
        const long long rounds = strips * two >= 128 ? two : one;
        if (s > rounds) s = rounds;
        const long long by_bytes = (long long)(0.015 * p.K / (p.M > 0 ? p.M : 1));
        if (s > by_bytes) s = by_bytes;
        if (s > 64) s = 64;
    }
    return s < 2 ? 1 : (int)s;
}

// Rows of K per slice (a multiple of 16) and the resulting slice count.
template <int Q, int WK, int U>
int rows_kslice(const Problem &p, int want, int *slices) {
    const int s = rows_slices<Q, WK, U>(p, want);
    const int kslice = 16 * (int)(((p.K + 15) / 16 + s - 1) / s);
    *slices = s == 1 ? 1 : (p.K + kslice - 1) / kslice;
    return *slices == 1 ? 16 * ((p.K + 15) / 16) : kslice;
}

// Columns per strip of a few-rows launch with `slices` K slices.  A
// workgroup of these kernels streams about 20-25 GB/s (one per CU), so a
// launch whose workgroups are fewer than the CUs, each reading a large share
// of B, leaves CUs idle and ends when the slowest workgroup does:
// 16 x 14336 x 4096 with B stored N x K in 64-row strips is 224 workgroups
// of 1 MB for 256 CUs.  With B stored transposed and large (32 MB or more)
// the strips are narrowed so that strips x slices comes as close to the CU
// count as a width that is a multiple of 4 allows (56 rows: 256 workgroups
// of 0.92 MB; graph-replayed 53.3 -> 48.7 us, 16 x 11008 x 4096 42.2 ->
// 38.7 us); lanes past a strip's width load nothing.  A strip of untransposed
// B is a run of each of its rows, and a width that is not a multiple of 32
// floats splits 128-byte lines between strips that both fetch them: narrowed
// that way 16 x 14336 x 4096 ran 44 -> 54 us, so those strips keep the
// tile's width.
constexpr int kRowsCUs = 256;
template <int Q, int WK, int U>
int rows_width(const Problem &p, int slices) {
    using S = RowsShape<Q, WK, U>;
    const long long strips = (p.N + S::COLS - 1) / S::COLS;
    if (!p.trans_b || p.batch != 1 || strips * slices >= kRowsCUs ||
        4LL * p.K * p.N < (32LL << 20))
        return S::COLS;
    const long long want = kRowsCUs / slices;   // strips
    const long long w = 4 * ((p.N + 4 * want - 1) / (4 * want));
    return w < S::COLS ? (int)w : S::COLS;
}

template <int Q, int WK, int U>
int rows_slice_count(const Problem &p, int group_m) {
    int slices = 1;
    rows_kslice<Q, WK, U>(p, group_m, &slices);
    return slices;
}

template <int Q, int WK, int U>
size_t rows_workspace(const Problem &p, int group_m) {
    int slices = 1;
    rows_kslice<Q, WK, U>(p, group_m, &slices);
    return slices == 1 ? 0 : (size_t)slices * p.M * p.N * 4;
}

// ST: the LDS-staged kernel for B stored transposed (Q = 1, WK = 4, U = 4,
// 16-byte rows of A and B).
template <int Q, int WK, int U, bool VA, bool VB, bool TA, bool TB, int IN = 0, bool ST = false>
hipError_t launch_rows_as(const Problem &p, int want_slices, hipStream_t stream) {
    using S = RowsShape<Q, WK, U>;
    static_assert(!ST || (Q == 1 && WK == 4 && U == 4 && VA && VB && TB && !TA),
                  "staged kernel: 64 columns, 4 waves, A and B^T in 16-byte rows");
    auto launch = [&](dim3 grid_dim, const RowsGrid &grid) {
        if constexpr (ST)
            hipLaunchKernelGGL((rows_tb_staged_kernel<WK, IN>), grid_dim, dim3(S::NT), 0, stream,
                               p, grid);
        else
            hipLaunchKernelGGL((rows_kernel<Q, WK, U, VA, VB, TA, TB, IN>), grid_dim, dim3(S::NT),
                               0, stream, p, grid);
    };
    RowsGrid grid{0, S::COLS, 1, 0, nullptr, nullptr};
    grid.kslice = rows_kslice<Q, WK, U>(p, want_slices, &grid.slices);
    grid.width = rows_width<Q, WK, U>(p, grid.slices);
    grid.strips = (p.N + grid.width - 1) / grid.width;
    if (grid.slices == 1) {
        launch(dim3(grid.strips, p.batch), grid);
        return hipGetLastError();
    }
    Workspace w;
    hipError_t e = workspace_acquire(rows_workspace<Q, WK, U>(p, want_slices), stream, p, w);
    if (e != hipSuccess) return e;
    grid.part = static_cast<float *>(w.ptr);
    grid.count = w.counters;
    launch(dim3(grid.strips * grid.slices), grid);
    e = hipGetLastError();
    const hipError_t f = workspace_release(w, stream);
    return e != hipSuccess ? e : f;
}

template <int Q, int WK, int U, bool TA, bool TB>
hipError_t launch_rows_ab(const Problem &p, int groups, bool va, bool vb, hipStream_t stream) {
    if constexpr (Q == 1 && WK == 4 && U == 4 && TB && !TA) {
        // A and B^T in 16-byte rows: staged through LDS (256-byte row runs per load)
        if (va && vb) return launch_rows_as<1, 4, 4, true, true, false, true, 0, true>(p, groups, stream);
    }
    if (va && vb) return launch_rows_as<Q, WK, U, true, true, TA, TB>(p, groups, stream);
    if (va) return launch_rows_as<Q, WK, U, true, false, TA, TB>(p, groups, stream);
    if (vb) return launch_rows_as<Q, WK, U, false, true, TA, TB>(p, groups, stream);
    return launch_rows_as<Q, WK, U, false, false, TA, TB>(p, groups, stream);
}

// VEC: 16-byte loads wherever an operand allows them (decided per operand:
// rows 16-byte aligned and the stored row length a multiple of 4); otherwise
// 4-byte loads throughout.  group_m, when positive, asks for that many K
// slices.
bool col1_applies(const Problem &p);
template <int IN>
hipError_t launch_col1(const Problem &p, hipStream_t stream);

// One row of C with B stored transposed (x W^T, W N x K) is, transposed, one
// column: C^T = W x^T, W's rows as the rows of A and x as the column, C's row
// as a column with unit row stride.  Run that way (the one-column kernel)
// when the library picks the K split, there is no bias (a bias per column of
// C would be one per row there) and the operands allow it.
Problem one_row_as_column(const Problem &p) {
    Problem q = p;
    q.M = p.N;
    q.N = 1;
    q.A = p.B;
    q.lda = p.ldb;
    q.stride_a = p.stride_b;
    q.B = p.A;
    q.ldb = p.lda;
    q.stride_b = p.stride_a;
    q.ldc = 1;
    return q;
}

// Whether a few-rows launch runs p as that column problem: one row, B
// stored transposed, no bias, the library's K split (group_m <= 0), 16-byte
// I/O (vec) and operands the one-column kernel takes.
bool takes_one_column(const Problem &p, int group_m, bool vec) {
    return vec && group_m <= 0 && p.M == 1 && p.trans_b && !p.trans_a && !p.bias &&
           col1_applies(one_row_as_column(p));
}

template <int Q, int WK, int U, bool VEC>
hipError_t launch_rows(const Problem &p, int group_m, hipStream_t stream) {
    if (takes_one_column(p, group_m, VEC)) return launch_col1<0>(one_row_as_column(p), stream);
    const bool va = VEC && !p.trans_a && rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) &&
                    p.K % 4 == 0;
    const bool vb = VEC && rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4) &&
                    (p.trans_b ? p.K : p.N) % 4 == 0;
    if (p.trans_a) {
        return p.trans_b ? launch_rows_ab<Q, WK, U, true, true>(p, group_m, false, vb, stream)
                         : launch_rows_ab<Q, WK, U, true, false>(p, group_m, false, vb, stream);
    }
    return p.trans_b ? launch_rows_ab<Q, WK, U, false, true>(p, group_m, va, vb, stream)
                     : launch_rows_ab<Q, WK, U, false, false>(p, group_m, va, vb, stream);
}

// ---------------------------------------------------------------- kind 1 ----
// One round of a wave's loads: U chunks of 256 k (lane l: k = 256 * chunk +
// 4l + 0..3): a[u][rr] = A(row rr, k .. k+3), b[u][j] = B(k .. k+3, column j).
template <int NB, int R, int U>
struct ColsRound {
    floatx4 a[U][R];
    floatx4 b[U][NB];
};

// BM (B's layout): 0 any K x N layout, read four bytes at a time; 1 a tight
// K x NB block (ldb == N == NB, 16-byte aligned, K a multiple of 4), so the
// 4*NB values of four consecutive k are contiguous and are read as NB 16-byte
// loads; 2 B stored transposed (N x K), each of its N rows read 16 bytes at a
// time like A's rows; 3 the same, four bytes at a time.  VA: 16-byte loads of
// A.  Each 256-k chunk gets resources of its own starting at its first k, so
// the per-lane offsets stay below 2^31: under R * lda floats for A, 256 * ldb
// for B, 16 * ldb for B^T.
template <int NB, int R, int U, bool VA, int BM>
__device__ __forceinline__ void cols_load(const Problem &p, int row0, int kc0, int lane,
                                          ColsRound<NB, R, U> &r) {
    const int ldb = (int)p.ldb, lda = (int)p.lda;
    const int rows = min(R, p.M - row0);
    const int kk = 4 * lane;   // this lane's first k of a chunk
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int kr = 256 * (kc0 + u);   // the chunk's first k (uniform)
        const int krem = p.K - kr;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(
            p.A + (long long)row0 * p.lda + kr, 4 * ((long long)(rows - 1) * p.lda + krem));
#pragma unroll
        for (int rr = 0; rr < R; ++rr) {
            const bool ok = rr < rows;
            if constexpr (VA) {
                r.a[u][rr] = ld4<true>(ra, (ok && kk < krem) ? (rr * lda + kk) * 4 : kOff);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r.a[u][rr][e] = ld1(ra, (ok && kk + e < krem) ? (rr * lda + kk + e) * 4 : kOff);
            }
        }
        if constexpr (BM >= 2) {
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(p.B + kr, 4 * ((long long)(p.N - 1) * p.ldb + krem));
#pragma unroll
            for (int jj = 0; jj < NB; ++jj) {
                const bool ok = jj < p.N;
                if constexpr (BM == 2) {
                    r.b[u][jj] = ld4<false>(rb, (ok && kk < krem) ? (jj * ldb + kk) * 4 : kOff);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        r.b[u][jj][e] = ld1(rb, (ok && kk + e < krem) ? (jj * ldb + kk + e) * 4 : kOff);
                }
            }
        } else {
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                p.B + (long long)kr * p.ldb, 4 * ((long long)(krem - 1) * p.ldb + p.N));
            if constexpr (BM == 1) {
                // B(kk + e, j) at float kk * NB + e * NB + j of the chunk
                floatx4 v[NB];
#pragma unroll
                for (int q = 0; q < NB; ++q)
                    v[q] = ld4<false>(rb, kk < krem ? (kk * NB + 4 * q) * 4 : kOff);
#pragma unroll
                for (int x = 0; x < 4 * NB; ++x) r.b[u][x % NB][x / NB] = v[x / 4][x % 4];
            } else {
#pragma unroll
                for (int jj = 0; jj < NB; ++jj) {
                    const bool ok = jj < p.N;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        r.b[u][jj][e] =
                            ld1(rb, (ok && kk + e < krem) ? ((kk + e) * ldb + jj) * 4 : kOff);
                }
            }
        }
    }
}

template <int NB, int R, int U>
__device__ __forceinline__ void cols_fma(const ColsRound<NB, R, U> &r, float (&acc)[R][NB]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int rr = 0; rr < R; ++rr)
#pragma unroll
                for (int jj = 0; jj < NB; ++jj)
                    acc[rr][jj] = fmaf(r.a[u][rr][e], r.b[u][jj][e], acc[rr][jj]);
}

// R rows of A per wave; rounds of U chunks double-buffered as in the
// few-rows kernel (chunks past K read as zero and touch no memory).
template <int NB, int R, int W, int U, bool VA, int BM>
__global__ void __launch_bounds__(64 * W) cols_kernel(Problem p) {
    select_batch(p);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int row0 = (blockIdx.x * W + wave) * R;
    if (row0 >= p.M) return;                      // whole wave leaves together; no barrier below
    float acc[R][NB];
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) acc[rr][jj] = 0.f;

    const int chunks = (p.K + 255) / 256;
    ColsRound<NB, R, U> r0, r1;
    cols_load<NB, R, U, VA, BM>(p, row0, 0, lane, r0);
    for (int kc = 0; kc < chunks; kc += 2 * U) {
        cols_load<NB, R, U, VA, BM>(p, row0, kc + U, lane, r1);
        pipeline_fence();
        cols_fma<NB, R, U>(r0, acc);
        if (kc + U >= chunks) break;
        cols_load<NB, R, U, VA, BM>(p, row0, kc + 2 * U, lane, r0);
        pipeline_fence();
        cols_fma<NB, R, U>(r1, acc);
    }
    // butterfly reduction over the 64 lanes (fixed order)
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
        for (int jj = 0; jj < NB; ++jj) {
            float v = acc[rr][jj];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            acc[rr][jj] = v;
        }
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
        if (row0 + rr >= p.M) break;
        float *crow = p.C + (long long)(row0 + rr) * p.ldc;
#pragma unroll
        for (int jj = 0; jj < NB; ++jj)
            if (lane == jj && jj < p.N) store_cell(p, crow + jj, jj, acc[rr][jj]);
    }
}

template <int NB, int R, int W, int U, bool VA, int BM>
hipError_t launch_cols_as(const Problem &p, hipStream_t stream) {
    const int blocks = (p.M + W * R - 1) / (W * R);
    hipLaunchKernelGGL((cols_kernel<NB, R, W, U, VA, BM>), dim3(blocks, p.batch), dim3(64 * W), 0,
                       stream, p);
    return hipGetLastError();
}

template <int NB, int R, int W, int U, int BM>
hipError_t launch_cols_bm(const Problem &p, bool va, hipStream_t stream) {
    return va ? launch_cols_as<NB, R, W, U, true, BM>(p, stream)
              : launch_cols_as<NB, R, W, U, false, BM>(p, stream);
}

// One column of C (N = 1) with A in 16-byte rows and the column of B a
// contiguous, 16-byte aligned vector x (B a tight K x 1 block, or its one row
// when stored transposed).  Wave w takes rows w, w + waves, ... in turn and
// streams them as one sequence of rounds of U chunks (1 KB of a row each),
// the next round's loads (of this row or the next) in flight while a round
// is multiplied, so the load pipeline does not drain between rows; one
// resource spans all of A (M * lda below 2^29 floats).  The C values that
// beta needs are read at the start, one per lane (a wave has at most 64
// rows), and reach lane 0 by a shuffle.  With 16-bit inputs (IN = 1, 2) the
// problem is in word form (K, lda, ldb count 32-bit words of two k values).
constexpr int kCol1Blocks = 512;

// acc + the dot product of four words of a row of A and of x: four floats
// (IN = 0), or eight 16-bit values in word form (IN = 1 bfloat16, 2 float16;
// the low half of a word holds the even k), each product exact in fp32.
template <int IN>
__device__ __forceinline__ float col1_dot(const floatx4 &a, const floatx4 &x, float acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (IN == 0) {
            acc = fmaf(a[e], x[e], acc);
        } else {
            const unsigned wa = __float_as_uint(a[e]), wx = __float_as_uint(x[e]);
            float al, ah, xl, xh;
            if constexpr (IN == 1) {
                al = __uint_as_float(wa << 16);
                ah = __uint_as_float(wa & 0xffff0000u);
                xl = __uint_as_float(wx << 16);
                xh = __uint_as_float(wx & 0xffff0000u);
            } else {
                al = (float)__builtin_bit_cast(_Float16, (unsigned short)(wa & 0xffffu));
                ah = (float)__builtin_bit_cast(_Float16, (unsigned short)(wa >> 16));
                xl = (float)__builtin_bit_cast(_Float16, (unsigned short)(wx & 0xffffu));
                xh = (float)__builtin_bit_cast(_Float16, (unsigned short)(wx >> 16));
            }
            acc = fmaf(al, xl, acc);
            acc = fmaf(ah, xh, acc);
        }
    }
    return acc;
}

template <int U, int IN>
__global__ void __launch_bounds__(256) col1_kernel(Problem p) {
    select_batch(p);
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = gridDim.x * 4;
    if (wid >= p.M) return;                       // whole wave leaves together; no barrier below
    const int lda = (int)p.lda, K = p.K;
    const int chunks = (K + 255) / 256, rpr = (chunks + U - 1) / U;   // rounds per row
    const int rows = (p.M - 1 - wid) / nw + 1, rounds = rows * rpr;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, 4 * ((long long)(p.M - 1) * p.lda + K));
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.B, 4LL * K);
    // C of this wave's row `lane` (beta != 0 only)
    const float cold = (p.beta != 0.f && lane < rows) ? p.C[(long long)(wid + lane * nw) * p.ldc]
                                                      : 0.f;
    auto issue = [&](int j, floatx4 (&a)[U], floatx4 (&x)[U]) {
        const bool ok = j < rounds;
        const int row = wid + (j / rpr) * nw, c0 = (j % rpr) * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (c0 + u) * 256 + 4 * lane;
            const bool in = ok && k < K;
            a[u] = ld4<true>(ra, in ? (row * lda + k) * 4 : kOff);
            x[u] = ld4<false>(rx, in ? k * 4 : kOff);
        }
    };
    float acc = 0.f;
    auto consume = [&](int j, const floatx4 (&a)[U], const floatx4 (&x)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) acc = col1_dot<IN>(a[u], x[u], acc);
        if (j % rpr == rpr - 1) {
            // butterfly reduction over the 64 lanes (fixed order)
            float v = acc;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            const int r = j / rpr;
            const float c = __shfl(cold, r, 64);
            if (lane == 0) {
                float out = p.alpha * v;
                if (p.beta != 0.f) out = fmaf(p.beta, c, out);
                if (p.has_epilogue()) out = activate(p.act, p.bias ? out + p.bias[0] : out);
                p.C[(long long)(wid + r * nw) * p.ldc] = out;
            }
            acc = 0.f;
        }
    };
    floatx4 a0[U], x0[U], a1[U], x1[U];
    issue(0, a0, x0);
    for (int j = 0; j < rounds; j += 2) {
        issue(j + 1, a1, x1);
        pipeline_fence();
        consume(j, a0, x0);
        if (j + 1 >= rounds) break;
        issue(j + 2, a0, x0);
        pipeline_fence();
        consume(j + 1, a1, x1);
    }
}

// Whether col1_kernel serves these operands (see there).
bool col1_applies(const Problem &p) {
    const bool x_vec = p.trans_b ? rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4)
                                 : p.ldb == 1 && rows_aligned(p.B, 4, p.stride_b, p.batch, 4);
    return p.N == 1 && !p.trans_a && p.K % 4 == 0 && x_vec &&
           rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) &&
           (long long)p.M * p.lda < (1LL << 29) && p.M <= 64LL * 4 * kCol1Blocks;
}

template <int IN>
hipError_t launch_col1(const Problem &p, hipStream_t stream) {
    const int blocks = min((p.M + 3) / 4, kCol1Blocks);
    hipLaunchKernelGGL((col1_kernel<4, IN>), dim3(blocks, p.batch), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// VEC: 16-byte loads of A where its rows allow them, and of B where it is one
// tight K x NB block or stored transposed with aligned rows (decided per
// operand; K a multiple of 4); otherwise 4-byte loads.  A stored transposed is
// not served.
template <int NB, int R, int W, int U, bool VEC>
hipError_t launch_cols(const Problem &p, int, hipStream_t stream) {
    if (p.trans_a) return hipErrorInvalidValue;
    if constexpr (NB == 1 && VEC) {
        if (col1_applies(p)) return launch_col1<0>(p, stream);
    }
    const bool k4 = p.K % 4 == 0;
    const bool va = VEC && k4 && rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4);
    const bool vb = VEC && k4 && rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4);
    if (p.trans_b)
        return vb ? launch_cols_bm<NB, R, W, U, 2>(p, va, stream)
                  : launch_cols_bm<NB, R, W, U, 3>(p, va, stream);
    // a tight K x NB block: 16-byte aligned, and so is every batch entry
    if (VEC && k4 && p.N == NB && p.ldb == NB && rows_aligned(p.B, 4, p.stride_b, p.batch, 4))
        return launch_cols_bm<NB, R, W, U, 1>(p, va, stream);
    return launch_cols_bm<NB, R, W, U, 0>(p, va, stream);
}

template <int Q, int WK, int U>
constexpr TileEntry rows_entry() {
    using S = RowsShape<Q, WK, U>;
    // the launchers apply a problem's bias / activation themselves, so the
    // 16-byte launcher is also the fused one; the LDS figure is the larger of
    // the register kernel's and, for the tile that also runs the LDS-staged
    // kernel (B stored transposed), that kernel's (all 160 KB)
    constexpr bool staged = Q == 1 && WK == 4 && U == 4;
    constexpr int lds = staged ? 2 * WK * kStagedFloats * 4 : S::LDS_BYTES;
    return TileEntry{{16, S::COLS, 16 * U, 16, S::COLS, 0, 0, S::NT, lds, 0, 0},
                     &launch_rows<Q, WK, U, true>, &launch_rows<Q, WK, U, false>, 0,
                     &launch_rows<Q, WK, U, true>};
}

template <int NB, int R, int W, int U>
constexpr TileEntry cols_entry() {
    return TileEntry{{W * R, NB, 256 * U, R, NB, 1, 0, 64 * W, 0, 0, 0},
                     &launch_cols<NB, R, W, U, true>, &launch_cols<NB, R, W, U, false>, 0,
                     &launch_cols<NB, R, W, U, true>};
}

// The few-rows tiles, in table order, with their workspace size functions.
#define SG_ROWS_TILES(X) X(2, 8, 1) X(2, 4, 2) X(1, 4, 2) X(1, 16, 1) X(1, 4, 4)

// 16-bit inputs, few rows: pw is the word-form problem (A untransposed, B
// transposed, K / lda / ldb in 32-bit words).
template <int IN>
hipError_t launch_rows16_as(const Problem &pw, hipStream_t stream) {
    const bool va = rows_aligned(pw.A, pw.lda, pw.stride_a, pw.batch, 4) && pw.K % 4 == 0;
    const bool vb = rows_aligned(pw.B, pw.ldb, pw.stride_b, pw.batch, 4) && pw.K % 4 == 0;
    // 16-byte rows: the LDS-staged kernel (256-byte runs of each weight row
    // per load, as for fp32)
    if (va && vb) return launch_rows_as<1, 4, 4, true, true, false, true, IN, true>(pw, 0, stream);
    return launch_rows_as<1, 8, 4, false, false, false, true, IN>(pw, 0, stream);
}

}  // namespace

hipError_t launch_skinny16(int dtype, const Problem &pw, hipStream_t stream) {
    if (pw.M > 16 || pw.trans_a || !pw.trans_b) return hipErrorInvalidValue;
    if (pw.M == 1 && !pw.bias) {
        // one row: the transposed one-column product, in word form
        const Problem q = one_row_as_column(pw);
        if (col1_applies(q))
            return dtype == SGEMM_DTYPE_BF16 ? launch_col1<1>(q, stream)
                                             : launch_col1<2>(q, stream);
    }
    return dtype == SGEMM_DTYPE_BF16 ? launch_rows16_as<1>(pw, stream)
                                     : launch_rows16_as<2>(pw, stream);
}

const TileEntry *skinny_tiles(int *count) {
#define SG_ROWS_ENTRY(Q, WK, U) rows_entry<Q, WK, U>(),
    static const TileEntry tiles[] = {
        SG_ROWS_TILES(SG_ROWS_ENTRY)   // 0-4: few rows (128-, 128-, 64-, 64-, 64-column strips)
        cols_entry<1, 2, 4, 4>(),      // 5-9: few columns
        cols_entry<2, 2, 4, 4>(),
        cols_entry<4, 2, 4, 2>(),
        cols_entry<8, 2, 4, 2>(),
        cols_entry<16, 2, 4, 1>(),
    };
#undef SG_ROWS_ENTRY
    *count = sizeof(tiles) / sizeof(tiles[0]);
    return tiles;
}

// K slices of a few-rows launch of `tile` with `group_m` asked-for slices
// (0: the library's choice); 1 for unsplit launches and kind 1.
int skinny_slices(int tile, const Problem &p, int group_m) {
    using SlFn = int (*)(const Problem &, int);
#define SG_ROWS_SL(Q, WK, U) &rows_slice_count<Q, WK, U>,
    static const SlFn fns[] = {SG_ROWS_TILES(SG_ROWS_SL)};
#undef SG_ROWS_SL
    constexpr int n = sizeof(fns) / sizeof(fns[0]);
    return (tile >= 0 && tile < n) ? fns[tile](p, group_m) : 1;
}

// Whether the few-rows launcher runs p (its library-chosen K split asked for
// with group_m <= 0) as the one-column product, which splits nothing.
bool skinny_one_row_column(const Problem &p, int group_m, bool vec) {
    return takes_one_column(p, group_m, vec);
}

// Workspace bytes of a few-rows launch of `tile` with `group_m` asked-for
// K slices (0: the library's choice); 0 for unsplit launches and kind 1.
size_t skinny_workspace_bytes(int tile, const Problem &p, int group_m) {
    using WsFn = size_t (*)(const Problem &, int);
#define SG_ROWS_WS(Q, WK, U) &rows_workspace<Q, WK, U>,
    static const WsFn fns[] = {SG_ROWS_TILES(SG_ROWS_WS)};
#undef SG_ROWS_WS
    constexpr int n = sizeof(fns) / sizeof(fns[0]);
    return (tile >= 0 && tile < n) ? fns[tile](p, group_m) : 0;
}

// The kind is recorded in the tile descriptor's tm field.
int skinny_kind(int tile) {
    int count = 0;
    const TileEntry *tiles = skinny_tiles(&count);
    return (tile >= 0 && tile < count) ? tiles[tile].desc.tm : -1;
}

// Kind 0 serves every transposition; kind 1 does not read A stored transposed.
// Both need the per-lane offsets of a chunk's resource below 2^31 bytes:
// kind 0 under 64 rows of B^T or 16 rows of B or A, kind 1 under its rows of
// A and 256 rows of B (16 of B^T).
bool skinny_fits(int tile, const Problem &p) {
    int count = 0;
    const TileEntry *tiles = skinny_tiles(&count);
    if (tile < 0 || tile >= count) return false;
    constexpr long long lim = 1LL << 29;   // floats
    if (skinny_kind(tile) == 0)
        return p.M <= 16 && 16 * p.lda < lim && (p.trans_b ? 64 : 16) * p.ldb < lim;
    return p.N <= tiles[tile].desc.bn && !p.trans_a && tiles[tile].desc.wm * p.lda < lim &&
           (p.trans_b ? 16 : 256) * p.ldb < lim;
}

namespace {

// Few-rows tile choice (measured with operands rotated past the Infinity
// Cache, graph-replayed): B stored transposed with 16-byte rows, the
// LDS-staged 64-column tile; otherwise 128-column strips of 8 waves where
// many rows of A would otherwise be re-read per 64 columns of B (M > 4, wide
// N); 64-column strips otherwise, 16 waves for narrow products (few strips,
// split deeply) and 4 waves (several workgroups per CU) for the rest.  Few columns: the
// narrowest tile that holds N.
int choose_skinny(const Problem &p) {
    const int M = p.M, N = p.N;
    if (M <= 16) {
        // B stored N x K in 16-byte rows (and A too): the LDS-staged kernel
        // (16 x 14336 x 4096: 49.6 us against 54.9 for the 64-column tile
        // loading B^T straight into registers)
        if (p.trans_b && !p.trans_a && p.K % 4 == 0 &&
            rows_aligned(p.A, p.lda, p.stride_a, p.batch, 4) &&
            rows_aligned(p.B, p.ldb, p.stride_b, p.batch, 4))
            return 4;
        if (!p.trans_b && M > 4 && N >= 8192) return 0;
        return N <= 2048 ? 3 : 2;
    }
    if (N <= 16 && !p.trans_a) {
        int count = 0;
        const TileEntry *tiles = skinny_tiles(&count);
        for (int t = 0; t < count; ++t)
            if (skinny_kind(t) == 1 && N <= tiles[t].desc.bn) return t;
    }
    return -1;
}

}  // namespace

// The skinny tile for a shape, or -1 when the family does not serve it.
int skinny_pick(const Problem &p) {
    const int t = choose_skinny(p);
    return skinny_fits(t, p) ? t : -1;
}

}  // namespace sg
