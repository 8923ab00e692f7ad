// scale.hip -- C = act(beta * C + bias): the alpha == 0 / K == 0 case of
// SGEMM, and the bias/activation pass for kernels that do not apply them in
// their own epilogue.
//
// With no product term left, C = alpha*(A*B) + beta*C reduces to scaling C
// ("a CUDA matmul" section 00 gives the full form).  beta == 0 writes without
// reading C, so NaN or Inf already in C does not survive.  bias (one float
// per column) and the activation are the optional epilogue of a linear layer
// ("The GEMM Scrapbook", introduction: the GEMMs of a feed-forward block).
#include "gemm_internal.hpp"

namespace sg {
namespace {

// Grid (x: column blocks, y: row bands, z: batch entries); lanes walk the
// columns so that neighbouring lanes touch neighbouring addresses.
__global__ void __launch_bounds__(256) elementwise_kernel(int M, int N, float beta, float *C,
                                                          long long ldc, long long stride_c,
                                                          const float *bias, int act) {
    C += (long long)blockIdx.z * stride_c;
    for (int i = blockIdx.y; i < M; i += gridDim.y) {
        float *row = C + (long long)i * ldc;
        for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < N; j += gridDim.x * blockDim.x) {
            float v = (beta == 0.f) ? 0.f : beta * row[j];
            if (bias) v += bias[j];
            row[j] = activate(act, v);
        }
    }
}

}  // namespace

hipError_t launch_elementwise(const Problem &p, float beta, hipStream_t stream) {
    const int bx = (p.N + 255) / 256 < 64 ? (p.N + 255) / 256 : 64;
    const int rows_per_entry = p.batch > 1 ? (4096 + p.batch - 1) / p.batch : 65535;
    const int by = p.M < rows_per_entry ? p.M : (rows_per_entry > 0 ? rows_per_entry : 1);
    for (int b0 = 0; b0 < p.batch; b0 += kMaxBatchPerLaunch) {
        const int nb = p.batch - b0 < kMaxBatchPerLaunch ? p.batch - b0 : kMaxBatchPerLaunch;
        hipLaunchKernelGGL(elementwise_kernel, dim3(bx, by, nb), dim3(256), 0, stream, p.M, p.N,
                           beta, p.C + (long long)b0 * p.stride_c, p.ldc, p.stride_c, p.bias,
                           p.act);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sg
