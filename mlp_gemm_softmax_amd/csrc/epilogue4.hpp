// Fused GEMM epilogues applied to four consecutive output columns at once
// (16-byte f32 / 8-byte bf16 vector accesses), shared by the large-tile
// bf16 kernel and the split-K epilogue kernel.
#pragma once

#include "kernels.hpp"
#include "optim_rule.hpp"

namespace mlp {

// Fused epilogue on four consecutive columns col..col+3 of one row (the
// column count is a multiple of 8, so all four are inside or all outside).
// `pre` is what epilogue_load fetched for the same place.
struct Pre {
    float4v w;        // Sgd, Adapt: the f32 master weights
    uint32_t m;       // MaskMul: four mask bytes
    float4v m1, m2;   // Adapt: first and second moments
};

template <Epi EPI>
__device__ __forceinline__ Pre epilogue_load(const GemmParams& p, int row, int col) {
    Pre pre{};
    const int64_t o = (int64_t)row * p.ldc + col;
    if constexpr (EPI == Epi::Sgd || EPI == Epi::Adapt) pre.w = *reinterpret_cast<const float4v*>(p.C + o);
    if constexpr (EPI == Epi::Adapt) {
        pre.m1 = *reinterpret_cast<const float4v*>(p.m + o);
        pre.m2 = *reinterpret_cast<const float4v*>(p.v + o);
    }
    if constexpr (EPI == Epi::MaskMul) pre.m = *reinterpret_cast<const uint32_t*>(p.mask + o);
    return pre;
}

typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2v pack_bf16x4(float4v v) {
    u32x2v r;
    r[0] = pack2_bf16(v[0], v[1]);
    r[1] = pack2_bf16(v[2], v[3]);
    return r;
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
            a[c] = relu_value(v[c]);
            m |= (pos ? 1u : 0u) << (8 * c);
        }
        // the next launch reads the activations, so they stay cached; the
        // mask is read only in the backward pass: streaming store
        if (p.Cb) *reinterpret_cast<u32x2v*>(p.Cb + o) = pack_bf16x4(a);
        else *reinterpret_cast<float4v*>(p.C + o) = a;
        __builtin_nontemporal_store(m, reinterpret_cast<uint32_t*>(p.mask + o));
    } else if constexpr (EPI == Epi::MaskMul) {
        float4v g;
#pragma unroll
        for (int c = 0; c < 4; ++c) g[c] = ((pre.m >> (8 * c)) & 0xffu) ? v[c] : 0.f;
        // streaming stores: measured faster for the whole step although the
        // next products read this gradient
        if (p.Cb) __builtin_nontemporal_store(pack_bf16x4(g), reinterpret_cast<u32x2v*>(p.Cb + o));
        else __builtin_nontemporal_store(g, reinterpret_cast<float4v*>(p.C + o));
    } else if constexpr (EPI == Epi::Sgd) {
        float4v w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = pre.w[c] - p.lr * v[c];
        *reinterpret_cast<float4v*>(p.C + o) = w;
        if (p.Cb) *reinterpret_cast<u32x2v*>(p.Cb + o) = pack_bf16x4(w);
    } else if constexpr (EPI == Epi::Adapt) {
        float4v w = pre.w, m1 = pre.m1, m2 = pre.m2;
        opt_apply4(p.opt, w, v, m1, m2);
        *reinterpret_cast<float4v*>(p.C + o) = w;
        *reinterpret_cast<float4v*>(p.m + o) = m1;
        *reinterpret_cast<float4v*>(p.v + o) = m2;
        if (p.Cb) *reinterpret_cast<u32x2v*>(p.Cb + o) = pack_bf16x4(w);
    }
}

}  // namespace mlp
