// Pointwise precision conversions of the bf16 fast path: float32 -> bfloat16
// (round to nearest even) for GEMM operands, and bfloat16 -> float32 for
// reading activations back.
#include "kernels.hpp"

namespace mlp {
namespace {

// Eight values per thread (two 16-byte loads in flight before either store)
// so that a single pass over a few tens of MB keeps enough bytes in flight.
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src,
                                                        bf16_t* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x * 8;
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i < n; i += stride) {
        if (i + 8 <= n) {
            const float4 v = *reinterpret_cast<const float4*>(src + i);
            const float4 w = *reinterpret_cast<const float4*>(src + i + 4);
            uint4 o;
            o.x = pack2_bf16(v.x, v.y);
            o.y = pack2_bf16(v.z, v.w);
            o.z = pack2_bf16(w.x, w.y);
            o.w = pack2_bf16(w.z, w.w);
            *reinterpret_cast<uint4*>(dst + i) = o;
        } else {
            for (size_t j = i; j < n; ++j) dst[j] = f32_to_bf16(src[j]);
        }
    }
}

__global__ __launch_bounds__(256) void widen_bf16_kernel(const bf16_t* __restrict__ src,
                                                         float* __restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = bf16_to_f32(src[i]);
}

int grid_for(size_t work) {
    size_t g = (work + 255) / 256;
    return (int)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

}  // namespace

hipError_t launch_cast_bf16(const float* src, bf16_t* dst, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for((n + 7) / 8)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

hipError_t launch_widen_bf16(const bf16_t* src, float* dst, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(widen_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace mlp
