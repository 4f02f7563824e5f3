// Fused GEMM epilogue applied to one float32 accumulator v at (row, col),
// shared by the tiled and small-product kernels (the vector form for the
// large-tile kernel is epilogue4.hpp).
#pragma once

#include "kernels.hpp"
#include "optim_rule.hpp"

namespace mlp {

template <Epi EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, int row, int col, float v) {
    const int64_t o = (int64_t)row * p.ldc + col;
    if constexpr (EPI == Epi::Store || EPI == Epi::Grad) {
        p.C[o] = v;
    } else if constexpr (EPI == Epi::ReluMask) {
        const bool pos = v > 0.f;
        const float a = relu_value(v);
        if (p.Cb) p.Cb[o] = f32_to_bf16(a); else p.C[o] = a;
        p.mask[o] = pos ? 1 : 0;
    } else if constexpr (EPI == Epi::MaskMul) {
        const float g = p.mask[o] ? v : 0.f;
        if (p.Cb) p.Cb[o] = f32_to_bf16(g); else p.C[o] = g;
    } else if constexpr (EPI == Epi::Sgd) {
        const float w = p.C[o] - p.lr * v;
        p.C[o] = w;
        if (p.Cb) p.Cb[o] = f32_to_bf16(w);
    } else if constexpr (EPI == Epi::Adapt) {
        // Adam / LaProp with g = v; the moments share W's layout
        float w = p.C[o], m = p.m[o], s = p.v[o];
        opt_apply(p.opt, w, v, m, s);
        p.C[o] = w;
        p.m[o] = m;
        p.v[o] = s;
        if (p.Cb) p.Cb[o] = f32_to_bf16(w);
    }
}

}  // namespace mlp
