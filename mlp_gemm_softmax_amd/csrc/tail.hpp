// Tail of the fused output layer (README "Example": the update of w2 and the
// mean of cross_entropy_loss), as a device function that any workgroup of
// NW waves can run: job j < ceil(H/16) computes rows 16j..16j+15 of
//   dW_L[h][c] = sum_b a[b][h] dlogits[b][c]
// on v_mfma_f32_16x16x4f32 (the waves split the batch rows; their sums meet
// in LDS and are added in wave order), then W_L -= lr * dW_L, an Adam /
// LaProp step, or a store of dW_L; job ceil(H/16) averages the row losses.  Every output belongs to
// one job, so no cross-workgroup reduction is needed; the head's writes are
// visible because the tail runs in a later launch.
#pragma once

#include "kernels.hpp"
#include "optim_rule.hpp"

namespace mlp {

// `red` is LDS scratch of at least NW * 2 * 64 float4.
template <int NW>
__device__ __forceinline__ void tail_job(const TailParams& t, int job, float4v* red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const int HB = (t.H + 15) / 16;
    if (job < HB) {
        const int h0 = 16 * job;
        const int CB = (t.C + 15) / 16;   // 1 or 2 (C <= 32)
        const int bpart = ((t.B + 4 * NW - 1) / (4 * NW)) * 4;
        const int bbeg = wave * bpart, bend = min(t.B, bbeg + bpart);
        float4v acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int hc = min(h0 + li, t.H - 1);
        // 8 steps of 4 rows at a time: the loads of all 8 (clamped in-range
        // addresses) go out before the first MFMA; out-of-range values are
        // zeroed where they are multiplied
        for (int k0 = bbeg; k0 < bend; k0 += 32) {
            float av[8], zv[8][2];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int b = min(k0 + 4 * u + lk, t.B - 1);
                av[u] = t.A[(int64_t)b * t.H + hc];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) zv[u][cb] = t.dZ[(int64_t)b * t.C + min(16 * cb + li, t.C - 1)];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int b = k0 + 4 * u + lk;
                const bool bok = b < bend;
                const float a = (bok && h0 + li < t.H) ? av[u] : 0.f;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    if (cb < CB) {
                        const float z = (bok && 16 * cb + li < t.C) ? zv[u][cb] : 0.f;
                        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, z, acc[cb], 0, 0, 0);
                    }
                }
            }
        }
        red[(wave * 2 + 0) * 64 + lane] = acc[0];
        red[(wave * 2 + 1) * 64 + lane] = acc[1];
        __syncthreads();
        if (wave < CB) {
            const int cb = wave;
            float4v d = red[cb * 64 + lane];
            for (int w = 1; w < NW; ++w) d += red[(w * 2 + cb) * 64 + lane];
            const int c = 16 * cb + li;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int h = h0 + 4 * lk + e;
                if (h < t.H && c < t.C) {
                    const int64_t o = (int64_t)h * t.C + c;
                    if (t.dW) {
                        t.dW[o] = d[e];
                    } else if (t.m) {
                        float w = t.W[o], m = t.m[o], s = t.v[o];
                        opt_apply(t.opt, w, d[e], m, s);
                        t.W[o] = w;
                        t.m[o] = m;
                        t.v[o] = s;
                    } else {
                        t.W[o] = t.W[o] - t.lr * d[e];
                    }
                }
            }
        }
    } else {
        // mean loss in a fixed order: per thread (8 loads in flight), a wave
        // butterfly, then the waves in order
        float s = 0.f;
        for (int b0 = tid; b0 < t.B; b0 += 8 * NW * 64) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = t.rowloss[min(b0 + u * NW * 64, t.B - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += b0 + u * NW * 64 < t.B ? v[u] : 0.f;
        }
        s = wave_sum(s);
        float* rs = reinterpret_cast<float*>(red);
        if (lane == 0) rs[wave] = s;
        __syncthreads();
        if (tid == 0) {
            float tot = 0.f;
            for (int w = 0; w < NW; ++w) tot += rs[w];
            *t.loss = tot * t.inv_b;
        }
    }
}

}  // namespace mlp
