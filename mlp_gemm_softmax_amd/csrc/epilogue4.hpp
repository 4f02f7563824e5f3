// Fused GEMM epilogues applied to four consecutive output columns at once
// (16-byte f32 / 8-byte bf16 vector accesses), shared by the large-tile
// bf16 kernel and the split-K epilogue kernel.
#pragma once

#include "kernels.hpp"

namespace mlp {

// Fused epilogue on four consecutive columns col..col+3 of one row (the
// column count is a multiple of 8, so all four are inside or all outside).
// `pre` is what epilogue_load fetched for the same place.
struct Pre {
    float4v w;        // Sgd: the f32 master weights
    uint32_t m;       // MaskMul: four mask bytes
};

template <Epi EPI>
__device__ __forceinline__ Pre epilogue_load(const GemmParams& p, int row, int col) {
    Pre pre{};
    const int64_t o = (int64_t)row * p.ldc + col;
    if constexpr (EPI == Epi::Sgd) pre.w = *reinterpret_cast<const float4v*>(p.C + o);
    if constexpr (EPI == Epi::MaskMul) pre.m = *reinterpret_cast<const uint32_t*>(p.mask + o);
    return pre;
}

__device__ __forceinline__ uint2 pack_bf16x4(float4v v) {
    return make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                      (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
}

template <Epi EPI>
__device__ __forceinline__ void epilogue4(const GemmParams& p, int row, int col, float4v v, const Pre& pre) {
    const int64_t o = (int64_t)row * p.ldc + col;
    if constexpr (EPI == Epi::Store || EPI == Epi::Grad) {
        *reinterpret_cast<float4v*>(p.C + o) = v;
    } else if constexpr (EPI == Epi::ReluMask) {
        uint32_t m = 0;
        float4v a;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bool pos = v[c] > 0.f;
            a[c] = pos ? v[c] : 0.f;
            m |= (pos ? 1u : 0u) << (8 * c);
        }
        if (p.Cb) *reinterpret_cast<uint2*>(p.Cb + o) = pack_bf16x4(a);
        else *reinterpret_cast<float4v*>(p.C + o) = a;
        *reinterpret_cast<uint32_t*>(p.mask + o) = m;
    } else if constexpr (EPI == Epi::MaskMul) {
        float4v g;
#pragma unroll
        for (int c = 0; c < 4; ++c) g[c] = ((pre.m >> (8 * c)) & 0xffu) ? v[c] : 0.f;
        if (p.Cb) *reinterpret_cast<uint2*>(p.Cb + o) = pack_bf16x4(g);
        else *reinterpret_cast<float4v*>(p.C + o) = g;
    } else if constexpr (EPI == Epi::Sgd) {
        float4v w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = pre.w[c] - p.lr * v[c];
        *reinterpret_cast<float4v*>(p.C + o) = w;
        if (p.Cb) *reinterpret_cast<uint2*>(p.Cb + o) = pack_bf16x4(w);
    }
}

}  // namespace mlp
