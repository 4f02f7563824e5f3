// Zeroing of the adaptive update rules' moments (mlp_set_optimizer), as a
// kernel.  The rules themselves (optim_rule.hpp) run inside the dW launches:
// every dW epilogue (Epi::Adapt), the skinny-batch passes and the output
// layer's tail apply Adam or LaProp while they hold W.
#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void zero_kernel(float4v* __restrict__ p, int64_t n4) {
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads)
        p[i] = z;
}

}  // namespace

hipError_t launch_zero(float* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    if (n % 4 || ((uintptr_t)p & 15u)) return hipErrorInvalidValue;
    const int64_t n4 = (int64_t)(n / 4);
    int64_t g = (n4 + kThreads - 1) / kThreads;
    g = g < 1 ? 1 : (g > 4096 ? 4096 : g);
    hipLaunchKernelGGL(zero_kernel, dim3((int)g), dim3(kThreads), 0, s, reinterpret_cast<float4v*>(p), n4);
    return hipGetLastError();
}

}  // namespace mlp
