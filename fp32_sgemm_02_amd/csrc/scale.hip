// scale.hip -- C = beta * C, the alpha == 0 / K == 0 case of SGEMM.
//
// With no product term left, C = alpha*(A*B) + beta*C reduces to scaling C
// ("a CUDA matmul" section 00 gives the full form).  beta == 0 writes zeros
// without reading C, so NaN or Inf already in C does not survive.
#include "gemm_internal.hpp"

namespace sg {
namespace {

// One workgroup row per C row band; lanes walk the columns so that neighbouring
// lanes touch neighbouring addresses.
__global__ void __launch_bounds__(256) scale_kernel(int M, int N, float beta, float *C,
                                                    long long ldc) {
    for (int i = blockIdx.y; i < M; i += gridDim.y) {
        float *row = C + (long long)i * ldc;
        for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < N; j += gridDim.x * blockDim.x)
            row[j] = (beta == 0.f) ? 0.f : beta * row[j];
    }
}

}  // namespace

hipError_t launch_scale(int M, int N, float beta, float *C, long long ldc, hipStream_t stream) {
    const int bx = (N + 255) / 256 < 64 ? (N + 255) / 256 : 64;
    const int by = M < 65535 ? M : 65535;
    hipLaunchKernelGGL(scale_kernel, dim3(bx, by), dim3(256), 0, stream, M, N, beta, C, ldc);
    return hipGetLastError();
}

}  // namespace sg
