// Split-K epilogue for the large-tile bf16 GEMM: adds the float32 partial
// sums of the K splits, [split][M][N] row-major, in split order and applies
// the product's fused epilogue.  A separate launch over all CUs: the last
// workgroup of each tile doing this inside the GEMM left three quarters of
// the CUs idle while it read every split's 256 KB tile back.
#include "epilogue4.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace mlp {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxSplits = 4;

template <Epi EPI>
__global__ __launch_bounds__(kThreads) void splitk_epilogue_kernel(GemmParams p) {
    const int64_t mn = (int64_t)p.M * p.N;
    const int64_t n4 = mn / 4;   // N is a multiple of 4
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
        const int64_t e = 4 * i;
        const int row = (int)(e / p.N), col = (int)(e % p.N);
        float4v v[kMaxSplits];
#pragma unroll
        for (int t = 0; t < kMaxSplits; ++t)   // splits past the last re-read it and are dropped
            v[t] = *reinterpret_cast<const float4v*>(p.partials + min(t, p.splits - 1) * mn + e);
        const Pre pre = epilogue_load<EPI>(p, row, col);
        float4v s = v[0];
#pragma unroll
        for (int t = 1; t < kMaxSplits; ++t)
            if (t < p.splits) s += v[t];
        epilogue4<EPI>(p, row, col, s, pre);
    }
}

template <Epi EPI>
hipError_t go(const GemmParams& p, hipStream_t st) {
    const int64_t n4 = (int64_t)p.M * p.N / 4;
    const int grid = (int)std::min<int64_t>((n4 + kThreads - 1) / kThreads, 2048);
    hipLaunchKernelGGL(splitk_epilogue_kernel<EPI>, dim3(grid), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_epilogue(const GemmParams& p, Epi epi, hipStream_t st) {
    if (p.splits < 2 || p.splits > kMaxSplits || p.N % 4 || p.ldc != p.N) return hipErrorInvalidValue;
    switch (epi) {
    case Epi::Store: return go<Epi::Store>(p, st);
    case Epi::ReluMask: return go<Epi::ReluMask>(p, st);
    case Epi::MaskMul: return go<Epi::MaskMul>(p, st);
    case Epi::Sgd: return go<Epi::Sgd>(p, st);
    case Epi::Grad: return go<Epi::Grad>(p, st);
    case Epi::Adapt: return go<Epi::Adapt>(p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace mlp
