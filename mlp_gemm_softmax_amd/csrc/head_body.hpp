// Body of the fused output layer for one block of batch rows (logits,
// softmax cross-entropy, dX of the last layer; README "Example": logits =
// matmul(h, w2) feeding cross_entropy_loss and the backward autodiff derives
// for them), shared by the stand-alone head kernel and the forward kernel
// that runs it in the workgroup finishing a row block's last column tile.
//
// W_L [H][C] and the rows' activations, labels and masks are staged in LDS
// (`lds`, head_lds_bytes(H, C, RB) bytes), then
//   logits[b][c] = sum_h a[b][h] W[h][c]
//   softmax-CE, 16 lanes per row -> dlogits, row loss
//   G[b][h] = mask[b][h] * sum_c dlogits[b][c] W[h][c]
// The two products run as 16x16 blocks on v_mfma_f32_16x16x4f32 with
// operands read from LDS (zero past the edges).  COH: the activations and
// masks were written in this launch by other workgroups with device-scope
// stores, so they are read with device-scope loads.  Needs kHeadThreads
// threads.
#pragma once

#include <math.h>

#include "kernels.hpp"

namespace mlp {

constexpr int kHeadThreads = 1024;
constexpr int kHeadWaves = kHeadThreads / kWave;
constexpr int kHeadU = 8;   // staging loads in flight per thread

template <bool COH>
__device__ __forceinline__ void head_block(const HeadParams& p, int row0, float* lds, float4v (*s_red)[kWave]) {
    const int H = p.H, C = p.C, CP = p.CP, RB = p.RB;
    const int HS = H | 1;             // odd LDS row stride: rows land on distinct banks
    float* sW = lds;                  // [H][CP]
    float* sA = sW + H * CP;          // [RB][HS]
    float* sZ = sA + RB * HS;         // [RB][C]  logits, then dlogits
    float* sT = sZ + RB * C;          // [RB][C]  labels
    uint8_t* sM = (uint8_t*)(sT + RB * C);   // [RB][H] mask
    const int tid = threadIdx.x;
    const int rows = min(RB, p.B - row0);

    // Stage everything the block reads once.  Loads go out kHeadU at a time per
    // thread from clamped (in-range) addresses before any is stored, so the
    // staging costs one memory round trip rather than one per element.
    {
        const float* gA = p.A + (int64_t)row0 * H;
        const uint8_t* gM = p.mask + (int64_t)row0 * H;
        const float* gT = p.labels + (int64_t)row0 * C;
        const int nA = rows * H, nW = H * C, nT = rows * C;
        for (int e0 = tid; e0 < nA; e0 += kHeadU * kHeadThreads) {
            float a[kHeadU];
            uint8_t m[kHeadU];
#pragma unroll
            for (int u = 0; u < kHeadU; ++u) {
                const int e = min(e0 + u * kHeadThreads, nA - 1);
                if constexpr (COH) {
                    a[u] = load_coherent(gA + e);
                    m[u] = load_coherent(gM + e);
                } else {
                    a[u] = gA[e];
                    m[u] = gM[e];
                }
            }
#pragma unroll
            for (int u = 0; u < kHeadU; ++u) {
                const int e = e0 + u * kHeadThreads;
                if (e < nA) {
                    sA[(e / H) * HS + e % H] = a[u];
                    sM[e] = m[u];
                }
            }
        }
        for (int e0 = tid; e0 < nW; e0 += kHeadU * kHeadThreads) {
            float w[kHeadU];
#pragma unroll
            for (int u = 0; u < kHeadU; ++u) w[u] = p.W[min(e0 + u * kHeadThreads, nW - 1)];
#pragma unroll
            for (int u = 0; u < kHeadU; ++u) {
                const int e = e0 + u * kHeadThreads;
                if (e < nW) sW[(e / C) * CP + e % C] = w[u];
            }
        }
        for (int e0 = tid; e0 < nT; e0 += kHeadU * kHeadThreads) {
            float t[kHeadU];
#pragma unroll
            for (int u = 0; u < kHeadU; ++u) t[u] = gT[min(e0 + u * kHeadThreads, nT - 1)];
#pragma unroll
            for (int u = 0; u < kHeadU; ++u) {
                const int e = e0 + u * kHeadThreads;
                if (e < nT) sT[e] = t[u];
            }
        }
    }
    __syncthreads();

    // logits Z = A W: 16x16 output blocks on v_mfma_f32_16x16x4f32 (the
    // K = H sum runs inside the matrix core, 4 h per step).  Operand lanes:
    // A[m = l%16][k = l/16], B[k = l/16][n = l%16]; the result lane l holds
    // rows 4(l/16)..+3 of column l%16.  The waves split each block's K range
    // into KS parts, whose sums meet in LDS and are added in part order.
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lk = lane >> 4;
    const int RBb = (rows + 15) / 16, CB = (C + 15) / 16, HB = (H + 15) / 16;
    {
        const int nb = RBb * CB;                       // <= 8 (RB <= 64, C <= 32)
        const int KS = kHeadWaves / nb >= 1 ? kHeadWaves / nb : 1;
        const int kpart = ((H + 4 * KS - 1) / (4 * KS)) * 4;
        if (wave < nb * KS) {
            const int blk = wave % nb, part = wave / nb;
            const int b0 = (blk / CB) * 16, c0 = (blk % CB) * 16;
            const int ba = b0 + li, cb = c0 + li;
            float4v acc = {0.f, 0.f, 0.f, 0.f};
            const int kb = part * kpart, ke = min(H, kb + kpart);
            for (int k0 = kb; k0 < ke; k0 += 4) {
                const int k = k0 + lk;
                const float av = (ba < rows && k < ke) ? sA[ba * HS + k] : 0.f;
                const float wv = (cb < C && k < ke) ? sW[k * CP + cb] : 0.f;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, wv, acc, 0, 0, 0);
            }
            s_red[wave][lane] = acc;
        }
        __syncthreads();
        if (wave < nb) {
            const int blk = wave;
            const int b0 = (blk / CB) * 16, c0 = (blk % CB) * 16;
            const int cb = c0 + li;
            float4v z = s_red[blk][lane];
            for (int part = 1; part < KS; ++part) z += s_red[part * nb + blk][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int bb = b0 + 4 * lk + e;
                if (bb < rows && cb < C) sZ[bb * C + cb] = z[e];
            }
        }
    }
    __syncthreads();

    // softmax cross-entropy, 16 lanes per row (classes j and j + 16 of the
    // row on lane j); max and sums by a fixed xor butterfly inside the
    // 16-lane group.  Only LDS is written before the next barrier (a barrier
    // also waits for the thread's outstanding global stores): the logits,
    // dlogits and row loss stay in this thread's registers and are stored
    // after the last phase.
    const int cb_row = tid >> 4, cj = tid & 15;
    const bool cv0 = cb_row < rows && cj < C, cv1 = cb_row < rows && cj + 16 < C;
    float cz0 = 0.f, cz1 = 0.f, cg0 = 0.f, cg1 = 0.f, closs = 0.f;
    {
        const int b = cb_row, j = cj;
        if (b < rows) {
            const float* t = sT + b * C;
            float* z = sZ + b * C;
            const bool v0 = cv0, v1 = cv1;
            const float z0 = v0 ? z[j] : -INFINITY, z1 = v1 ? z[j + 16] : -INFINITY;
            const float t0 = v0 ? t[j] : 0.f, t1 = v1 ? t[j + 16] : 0.f;
            float mx = fmaxf(z0, z1);
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
            const float e0 = v0 ? expf(z0 - mx) : 0.f, e1 = v1 ? expf(z1 - mx) : 0.f;
            float se = e0 + e1, st = t0 + t1, stz = (v0 ? t0 * z0 : 0.f) + (v1 ? t1 * z1 : 0.f);
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                se += __shfl_xor(se, o, 16);
                st += __shfl_xor(st, o, 16);
                stz += __shfl_xor(stz, o, 16);
            }
            const float lse = mx + logf(se);
            cz0 = z0;
            cz1 = z1;
            if (v0) {
                cg0 = (e0 / se * st - t0) * p.inv_b;
                z[j] = cg0;
            }
            if (v1) {
                cg1 = (e1 / se * st - t1) * p.inv_b;
                z[j + 16] = cg1;
            }
            closs = st * lse - stz;
        }
    }
    __syncthreads();

    // dX of the last layer through the ReLU mask: G = (dZ W^T) . m, blocks
    // of 16 rows x 16 h with K = C on the matrix core.
    for (int blk = wave; blk < RBb * HB; blk += kHeadThreads / kWave) {
        const int b0 = (blk / HB) * 16, h0 = (blk % HB) * 16;
        const int ba = b0 + li, hb = h0 + li;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < C; k0 += 4) {
            const int k = k0 + lk;
            const float zv = (ba < rows && k < C) ? sZ[ba * C + k] : 0.f;
            const float wv = (hb < H && k < C) ? sW[hb * CP + k] : 0.f;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(zv, wv, acc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int bb = b0 + 4 * lk + e;
            if (bb < rows && hb < H) p.G[(int64_t)(row0 + bb) * H + hb] = sM[bb * H + hb] ? acc[e] : 0.f;
        }
    }

    // the softmax-CE phase's outputs
    const int64_t o = (int64_t)(row0 + cb_row) * C + cj;
    if (cv0) {
        if (p.logits) p.logits[o] = cz0;
        p.dlogits[o] = cg0;
    }
    if (cv1) {
        if (p.logits) p.logits[o + 16] = cz1;
        p.dlogits[o + 16] = cg1;
    }
    if (cb_row < rows && cj == 0) p.rowloss[row0 + cb_row] = closs;
}

}  // namespace mlp
