// gemm_internal.hpp -- types shared by the kernels and the C-ABI dispatcher.
//
// Internal to the library: nothing here is exported.  The public interface is
// include/fp32_sgemm.h.
#pragma once

#include <hip/hip_runtime.h>

#include "fp32_sgemm.h"

namespace sg {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// One GEMM problem, C = alpha * (A * B) + beta * C, row-major with leading
// dimensions (in floats).  Offsets are formed in 64-bit inside the kernels.
struct Problem {
    int M, N, K;
    float alpha, beta;
    const float *A;
    long long lda;
    const float *B;
    long long ldb;
    float *C;
    long long ldc;
    int trans_a = 0;   // A stored transposed (K x M)
    int trans_b = 0;   // B stored transposed (N x K)
};

using LaunchFn = hipError_t (*)(const Problem &, int group_m, hipStream_t);

// One compiled tile configuration of a kernel family: a launcher for 16-byte
// vector I/O (all of A, B, C 16-byte aligned with leading dimensions that are
// multiples of 4) and one for 4-byte I/O (anything 4-byte aligned).
struct TileEntry {
    sgemm_tile_desc desc;
    LaunchFn vec;
    LaunchFn scalar;
    int eff_pct = 0;   // measured fraction of the fp32 peak at 4096^3 (dispatch cost model)
};

// Kernel families (each defined in its own .hip file): the compiled tile
// configurations, as a table owned by the family (host functions only).
const TileEntry *mfma_tiles(int *count);
const TileEntry *mfma_direct_tiles(int *count);      // direct-load tiles, A untransposed
const TileEntry *mfma_direct_ta_tiles(int *count);   // ... A transposed
bool direct_applies(const Problem &p, int bm, int bn, int bk, bool edges);
const TileEntry *valu_tiles(int *count);
const TileEntry *skinny_tiles(int *count);

// Skinny family: which entry serves a shape (-1 if none applies), and which
// orientation an entry serves (0: few rows of C, M <= 16; 1: few columns, N <= 16).
int skinny_pick(int M, int N, int K);
int skinny_kind(int tile);
bool skinny_fits(int tile, int M, int N);

// C = beta * C (beta == 0: zero fill without reading C).
hipError_t launch_scale(int M, int N, float beta, float *C, long long ldc,
                        hipStream_t stream);

// ---- device helpers shared by the families ---------------------------------

// Ends one software-pipeline step.  The accumulators pass through an empty
// asm statement, so the arithmetic of this step must be complete at this
// point; the memory clobber keeps the LDS reads issued for the next step from
// moving above it.  Without this the compiler sinks all the (side-effect
// free) arithmetic of a loop body below its loads and then needs registers
// for every step's operands at once.  The asm emits no instruction.
template <int N>
__device__ __forceinline__ void pipeline_fence(float (&acc)[N]) {
    static_assert(N % 4 == 0, "accumulators in groups of four");
#pragma unroll
    for (int i = 0; i < N; i += 4)
        asm volatile("" : "+v"(acc[i]), "+v"(acc[i + 1]), "+v"(acc[i + 2]), "+v"(acc[i + 3]));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Step boundary for the matrix-core kernels: memory ordering only.  The MFMA
// builtins are not moved across it by the compiler, so tying the
// accumulators (which would pin all of them to fixed registers at every step)
// is unnecessary there.
__device__ __forceinline__ void pipeline_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8), and each XCD has its own L2.  Renumber so that XCD x receives a
// contiguous range of logical tile ids; neighbouring tiles (which share rows
// of A or columns of B) then share an L2.  Bijective on [0, T) for any T.
__device__ __forceinline__ int xcd_remap(int w, int T) {
    constexpr int XCDS = 8;
    const int q = T / XCDS, r = T % XCDS;
    const int x = w % XCDS, l = w / XCDS;
    return x * q + (x < r ? x : r) + l;
}

// Logical tile id -> (tile row, tile column), walking blocks of `group_m`
// tile-rows column by column, so consecutive ids reuse the same B columns
// across group_m rows of A.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n,
                                            int group_m, int &tm, int &tn) {
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int rows = min(tiles_m - first_m, group_m);
    const int in_g = t - g * per_group;
    tm = first_m + in_g % rows;
    tn = in_g / rows;
}

}  // namespace sg
