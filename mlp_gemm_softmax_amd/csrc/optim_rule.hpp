// One element of the adaptive update rules (Adam: Kingma and Ba, "Adam: A
// Method for Stochastic Optimization", Algorithm 1; LaProp: Ziyin, Wang and
// Ueda, "LaProp: Separating Momentum and Adaptivity in Adam", Algorithm 1),
// in float32, shared by the multi-tensor update launch and the skinny-batch
// kernels that apply the rule while W streams through them.
#pragma once

#include "kernels.hpp"

namespace mlp {

__device__ __forceinline__ void opt_apply(const OptScalars& o, float& w, float g, float& m, float& v) {
    if (o.rule == kOptAdam) {
        m = o.b1 * m + o.om1 * g;
        v = o.b2 * v + o.om2 * (g * g);
        w = w - o.lr * (m * o.inv_c1) / (sqrtf(v * o.inv_c2) + o.eps);
    } else {
        v = o.b2 * v + o.om2 * (g * g);
        m = o.b1 * m + o.om1 * (g / (sqrtf(v * o.inv_c2) + o.eps));
        w = w - o.lr * (m * o.inv_c1);
    }
}

__device__ __forceinline__ void opt_apply4(const OptScalars& o, float4v& w, float4v g, float4v& m, float4v& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float we = w[e], me = m[e], ve = v[e];
        opt_apply(o, we, g[e], me, ve);
        w[e] = we;
        m[e] = me;
        v[e] = ve;
    }
}

}  // namespace mlp
