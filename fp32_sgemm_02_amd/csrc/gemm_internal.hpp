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
// A batch of `batch` such products runs in one launch: blockIdx.y is the
// product's index, and its operands start `stride_*` floats further per index.
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
    int batch = 1;
    long long stride_a = 0, stride_b = 0, stride_c = 0;
    const float *bias = nullptr;   // epilogue: one float per column of C, or none
    int act = SGEMM_ACT_NONE;      // epilogue activation
    // Device memory that partial sums of this call take instead of the
    // library's workspace (the entry point that allocates nothing): arrival
    // counters first (kWorkspaceCounterBytes, zero between launches), then
    // scratch_bytes for the sums.  Null: the workspace of workspace_acquire.
    void *scratch = nullptr;
    size_t scratch_bytes = 0;
    __host__ __device__ bool has_epilogue() const {
        return bias != nullptr || act != SGEMM_ACT_NONE;
    }
};

// A product with 16-bit A and B (bfloat16 or float16 bit patterns; sizes and
// leading dimensions in elements) and fp32 C, for the generic 16-bit kernel.
struct Problem16 {
    int M, N, K;
    float alpha, beta;
    const unsigned short *A;
    long long lda;
    const unsigned short *B;
    long long ldb;
    float *C;
    long long ldc;
    int trans_a = 0, trans_b = 0;
    int batch = 1;
    long long stride_a = 0, stride_b = 0, stride_c = 0;
};

// Largest grid y (batch entries per launch); larger batches are split.
constexpr int kMaxBatchPerLaunch = 65535;

// Host: whether every batch entry of an operand has rows starting on
// `floats`-float boundaries (base aligned, and the leading dimension and the
// batch stride multiples of `floats`).
inline bool rows_aligned(const void *ptr, long long ld, long long stride, int batch, int floats) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(ptr);
    return a % (4ull * floats) == 0 && ld % floats == 0 && (batch <= 1 || stride % floats == 0);
}

using LaunchFn = hipError_t (*)(const Problem &, int group_m, hipStream_t);

// One compiled tile configuration of a kernel family: a launcher for 16-byte
// vector I/O (all of A, B, C 16-byte aligned with leading dimensions that are
// multiples of 4) and one for 4-byte I/O (anything 4-byte aligned).
struct TileEntry {
    sgemm_tile_desc desc;
    LaunchFn vec;
    LaunchFn scalar;
    int eff_pct = 0;   // measured fraction of the fp32 peak at 4096^3 (dispatch cost model)
    // launcher that applies the problem's bias / activation in the kernel's
    // own epilogue (16-byte I/O); returns hipErrorNotSupported for operands
    // it does not serve, and the caller then adds an elementwise pass
    LaunchFn fused = nullptr;
    // stream-K launcher (persistent runs over split k-iterations and a
    // fixup); hipErrorNotSupported for operands it does not serve
    LaunchFn streamk = nullptr;
};

// Kernel families (each defined in its own .hip file): the compiled tile
// configurations, as a table owned by the family (host functions only).
const TileEntry *mfma_tiles(int *count);
const TileEntry *mfma_direct_tiles(int *count);      // direct-load tiles, A untransposed
const TileEntry *mfma_direct_ta_tiles(int *count);   // ... A transposed
// their fused-epilogue launchers, one per tile in table order
const LaunchFn *mfma_direct_epi_launchers(int *count);
const LaunchFn *mfma_direct_ta_epi_launchers(int *count);
// Device workspace of a launch that keeps partial sums (workspace.cpp): the
// problem's scratch when it has one; otherwise, outside graph capture, the
// buffer cached for the (device, stream), reused by every call on that
// stream; under capture a stream-ordered allocation of the graph's own.
// Every workspace starts with kWorkspaceCounters arrival counters, zero
// between launches (a launch that counts arrivals sets them back to zero),
// followed by `bytes` for the partial sums.  Release after the launches that
// use it.
constexpr int kWorkspaceCounters = 4096;
constexpr size_t kWorkspaceCounterBytes = 4 * kWorkspaceCounters;
struct Workspace {
    void *ptr = nullptr;            // the partial sums
    unsigned *counters = nullptr;   // kWorkspaceCounters arrival counters
    void *base = nullptr;           // the allocation (graph capture)
    bool owned = false;             // allocated for this call (graph capture)
};
hipError_t workspace_acquire(size_t bytes, hipStream_t stream, const Problem &p, Workspace &w);
hipError_t workspace_release(const Workspace &w, hipStream_t stream);
hipError_t workspace_release_all();   // the current device's cached buffers
// The static scratch array of the current device (workspace.cpp): its device
// address (counters first, as in a workspace) and the bytes after the counters.
hipError_t static_scratch(void **ptr, size_t *bytes);

// their stream-K launchers (null where a tile offers none), same order
const LaunchFn *mfma_direct_sk_launchers(int *count);
const LaunchFn *mfma_direct_ta_sk_launchers(int *count);
bool direct_applies(const Problem &p, int bm, int bn, int bk, bool edges);
const TileEntry *valu_tiles(int *count);
const TileEntry *skinny_tiles(int *count);

// 16-bit-input family (mfma_gemm16.hip): the direct-load MFMA tiles for A
// untransposed and B transposed, over the problem in 32-bit words along k, and
// the generic kernel for every layout.
int tiles16_count();
const sgemm_tile_desc *tile16_desc(int tile);
int tile16_eff(int tile);
hipError_t launch_tile16(int tile, int dtype, const Problem &pw, int group_m, hipStream_t stream);
hipError_t launch_generic16(int dtype, const Problem16 &p, hipStream_t stream);
// ... and the few-rows skinny kernel over the same word form (M <= 8).
hipError_t launch_skinny16(int dtype, const Problem &pw, hipStream_t stream);

// Skinny family: which entry serves a shape (-1 if none applies), and which
// orientation an entry serves (0: few rows of C, M <= 16; 1: few columns, N <= 16).
int skinny_pick(const Problem &p);
int skinny_kind(int tile);
bool skinny_fits(int tile, const Problem &p);
// Workspace bytes (after the counters) of a skinny launch of `tile`, with
// group_m as passed to its launcher; 0 when it needs none.
size_t skinny_workspace_bytes(int tile, const Problem &p, int group_m);
// K slices of a few-rows skinny launch (group_m as passed to its launcher).
int skinny_slices(int tile, const Problem &p, int group_m);
// Whether the few-rows launcher runs p (one row, B stored transposed, no
// bias; group_m as passed to it, vec: 16-byte I/O) as the one-column product,
// which splits nothing.
bool skinny_one_row_column(const Problem &p, int group_m, bool vec);

// Small-product family (small_gemm.hip): its tiles; whether it can run a
// problem (A untransposed, 31-bit offsets); the tile automatic dispatch
// gives a problem (-1: leave it to the tiled families); and its tile for a
// problem it is asked to run without a tile.
const TileEntry *small_tiles(int *count);
bool small_fits(const Problem &p);
int small_pick(const Problem &p);
bool small_tiny_batch(const Problem &p);   // a batch of tiny products (small family first)
int small_choice(const Problem &p);

// C = act(beta * C + bias) over p's batch (beta == 0: C is not read); with
// no epilogue, C = beta * C.  The alpha == 0 / K == 0 case, and the bias and
// activation pass after a kernel that does not apply them itself (beta = 1).
hipError_t launch_elementwise(const Problem &p, float beta, hipStream_t stream);

// ---- device helpers shared by the families ---------------------------------

// Moves the operand pointers to this workgroup's batch entry (blockIdx.y).
__device__ __forceinline__ void select_batch(Problem &p) {
    const long long b = blockIdx.y;
    p.A += b * p.stride_a;
    p.B += b * p.stride_b;
    p.C += b * p.stride_c;
}

// Activation of a finished sum (SGEMM_ACT_*), in fp32.  GELU's normal CDF is
// evaluated as erfc(-x / sqrt 2) / 2 and (1 + tanh u) / 2 as 1 / (1 + e^-2u):
// the same functions without the cancellation of 1 + erf and 1 + tanh at
// negative x.
template <int ACT>
__device__ __forceinline__ float activate_t(float x) {
    if constexpr (ACT == SGEMM_ACT_RELU) {
        return x < 0.f ? 0.f : x;
    } else if constexpr (ACT == SGEMM_ACT_SILU) {
        return x / (1.f + expf(-x));
    } else if constexpr (ACT == SGEMM_ACT_GELU_ERF) {
        return 0.5f * x * erfcf(-0.70710678118654752f * x);
    } else if constexpr (ACT == SGEMM_ACT_GELU_TANH) {
        const float u = 0.79788456080286536f * fmaf(0.044715f * x, x * x, x);
        return x / (1.f + expf(-2.f * u));
    } else {
        return x;
    }
}

__device__ __forceinline__ float activate(int act, float x) {
    switch (act) {
    case SGEMM_ACT_RELU: return activate_t<SGEMM_ACT_RELU>(x);
    case SGEMM_ACT_SILU: return activate_t<SGEMM_ACT_SILU>(x);
    case SGEMM_ACT_GELU_ERF: return activate_t<SGEMM_ACT_GELU_ERF>(x);
    case SGEMM_ACT_GELU_TANH: return activate_t<SGEMM_ACT_GELU_TANH>(x);
    default: return x;
    }
}

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
