// peak_probes.hip -- measured ceilings for the roofline denominators.
//
// Two register-only kernels that keep one execution unit busy and touch
// memory only to publish a result (so the work cannot be removed):
//   * probe_mfma_f32: chains of independent v_mfma_f32_16x16x4_f32 per wave;
//     2048 flops per instruction.
//   * probe_valu_f32: chains of independent fp32 FMAs per lane (built, like
//     the library, with packed fp32 disabled), 2 flops per lane per FMA.
//   * probe_read_f32: a plain streaming read, each workgroup one contiguous
//     chunk, 16-byte non-temporal loads, eight in flight per lane: the HBM
//     read rate a memory-bound kernel can reach with a given number of
//     workgroups (the roofline paragraph of "The GEMM Scrapbook" bounds such
//     kernels by bandwidth, not flops).
// The achieved rate divided by (256 CUs x 256 flops/clock) gives the
// effective matrix-core clock during a long fp32 MFMA run.  Not part of the
// SGEMM library: built into libfp32probes.so and used by bench.py --probes.
#include <hip/hip_runtime.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 16;

__global__ void __launch_bounds__(256) probe_mfma_kernel(int iters, float *out) {
    floatx4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
    const float a = 1e-3f * (threadIdx.x & 7), b = 1e-3f * (threadIdx.x >> 3);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
    }
    floatx4 s = acc[0];
#pragma unroll
    for (int c = 1; c < kChains; ++c) s += acc[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

__global__ void __launch_bounds__(256) probe_valu_kernel(int iters, float *out) {
    float acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = 1e-3f * c;
    const float a = 0.999f + 1e-6f * threadIdx.x, b = 1e-4f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = fmaf(acc[c], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Workgroup b reads floats [b * chunk, (b + 1) * chunk) of src (chunk a
// multiple of 4); lanes past the chunk load its first element and discard it
// (no branch around the loads, so all eight stay in flight together).  Each
// thread writes its sum, so the loads cannot be removed.
__global__ void __launch_bounds__(256) probe_read_kernel(const float *src, long long chunk,
                                                         float *out) {
    const floatx4 *p = reinterpret_cast<const floatx4 *>(src + (long long)blockIdx.x * chunk);
    const long long n4 = chunk / 4;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (long long i = threadIdx.x; i < n4; i += 256 * 8) {
        floatx4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long long j = i + 256LL * u;
            const bool ok = j < n4;
            const floatx4 t = __builtin_nontemporal_load(ok ? p + j : p);
            v[u] = ok ? t : floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

extern "C" {

// Streaming read of n floats by `blocks` workgroups of 256 threads; n must be
// a multiple of 4 * blocks and `out` hold blocks * 256 floats.  Returns a
// hipError_t, or -1 for a size that does not divide.
int probe_read_f32(const float *src, long long n, int blocks, float *out, hipStream_t stream) {
    if (blocks <= 0 || n <= 0 || n % (4LL * blocks) != 0) return -1;
    hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(256), 0, stream, src, n / blocks,
                       out);
    return (int)hipGetLastError();
}

// Flops performed by one launch of each probe with `blocks` workgroups of 256
// threads (4 waves) and `iters` iterations.
double probe_mfma_flops(int blocks, int iters) {
    return (double)blocks * 4 * iters * kChains * 2048.0;
}
double probe_valu_flops(int blocks, int iters) {
    return (double)blocks * 256 * iters * kChains * 2.0;
}

// `out` must hold blocks * 256 floats (device memory).  Returns a hipError_t.
int probe_mfma_f32(int blocks, int iters, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
    return (int)hipGetLastError();
}
int probe_valu_f32(int blocks, int iters, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(probe_valu_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
    return (int)hipGetLastError();
}

}  // extern "C"
