// Adaptive update rules (the README "Contents" names Adam and LaProp, whose
// moments a session allocates only on request): one launch updates every
// layer from the gradients the training step stored, elementwise, in float32.
//
//   Adam   (Kingma and Ba, "Adam: A Method for Stochastic Optimization",
//           Algorithm 1):
//             m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g^2
//             W <- W - lr (m / c1) / (sqrt(v / c2) + eps)
//   LaProp (Ziyin, Wang and Ueda, "LaProp: Separating Momentum and
//           Adaptivity in Adam", Algorithm 1):
//             v <- b2 v + (1 - b2) g^2
//             m <- b1 m + (1 - b1) g / (sqrt(v / c2) + eps)
//             W <- W - lr m / c1
// with c1 = 1 - b1^t, c2 = 1 - b2^t at step t (1/c1 and 1/c2 come in from
// the host, computed in double).  In the bf16 mode the operand copy of W is
// rewritten from the new master.  The update is bound by HBM traffic: per
// weight it reads g, m, v, W and writes m, v, W (+ the bf16 copy).
#include "kernels.hpp"
#include "optim_rule.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocksPerTensor = 2048;

__global__ __launch_bounds__(kThreads) void opt_update_kernel(OptParams p) {
    // tensor of this block (uniform scan over at most kMaxOptTensors entries)
    int ti = 0;
    while (ti + 1 < p.count && (int)blockIdx.x >= p.first_block[ti + 1]) ++ti;
    const OptTensor& t = p.t[ti];
    const int nb = p.first_block[ti + 1] - p.first_block[ti];
    const int64_t n4 = t.n / 4;
    const int64_t stride = (int64_t)nb * kThreads;
    for (int64_t i = (int64_t)(blockIdx.x - p.first_block[ti]) * kThreads + threadIdx.x; i < n4; i += stride) {
        float4v w = *reinterpret_cast<const float4v*>(t.W + 4 * i);
        const float4v g = *reinterpret_cast<const float4v*>(t.g + 4 * i);
        float4v m = *reinterpret_cast<const float4v*>(t.m + 4 * i);
        float4v v = *reinterpret_cast<const float4v*>(t.v + 4 * i);
        opt_apply4(p.o, w, g, m, v);
        *reinterpret_cast<float4v*>(t.W + 4 * i) = w;
        *reinterpret_cast<float4v*>(t.m + 4 * i) = m;
        *reinterpret_cast<float4v*>(t.v + 4 * i) = v;
        if (t.Wb) {
            uint2 h;
            h.x = (uint32_t)f32_to_bf16(w[0]) | ((uint32_t)f32_to_bf16(w[1]) << 16);
            h.y = (uint32_t)f32_to_bf16(w[2]) | ((uint32_t)f32_to_bf16(w[3]) << 16);
            *reinterpret_cast<uint2*>(t.Wb + 4 * i) = h;
        }
    }
    // the last n % 4 elements: first block of the tensor
    if (blockIdx.x == p.first_block[ti] && threadIdx.x < (t.n & 3)) {
        const int64_t j = 4 * n4 + threadIdx.x;
        float w = t.W[j], m = t.m[j], v = t.v[j];
        opt_apply(p.o, w, t.g[j], m, v);
        t.W[j] = w;
        t.m[j] = m;
        t.v[j] = v;
        if (t.Wb) t.Wb[j] = f32_to_bf16(w);
    }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(float4v* __restrict__ p, int64_t n4) {
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads)
        p[i] = z;
}

}  // namespace

hipError_t launch_opt_update(OptParams p, hipStream_t s) {
    if (p.count < 1 || p.count > kMaxOptTensors || (p.o.rule != kOptAdam && p.o.rule != kOptLaProp))
        return hipErrorInvalidValue;
    int blocks = 0;
    for (int i = 0; i < p.count; ++i) {
        const OptTensor& t = p.t[i];
        if (t.n < 1 || !t.W || !t.g || !t.m || !t.v) return hipErrorInvalidValue;
        p.first_block[i] = blocks;
        const int64_t want = (t.n / 4 + kThreads - 1) / kThreads;
        blocks += (int)(want < 1 ? 1 : (want > kMaxBlocksPerTensor ? kMaxBlocksPerTensor : want));
    }
    p.first_block[p.count] = blocks;
    hipLaunchKernelGGL(opt_update_kernel, dim3(blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

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
