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

// Sum / max over the 16 lanes of a DPP row, the result in every lane: pairs
// (quad_perm 1,0,3,2), quads (2,3,0,1), half rows (row_half_mirror), rows
// (row_mirror); a fixed order, plain VALU moves instead of LDS permutes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return v;
}

// q = e / d and e - q d for 0 <= e < 2^22, 1 <= d <= 2^16, from a float
// reciprocal (rinv = 1/d rounded): (e + 1/2)/d sits at least 1/(2d) away
// from an integer and the product errs by far less, so the floor is exact.
// Cheaper than the integer division sequence, which every lane would run.
__device__ __forceinline__ int div_small(int e, float rinv) { return (int)(((float)e + 0.5f) * rinv); }

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
    const float rH = 1.0f / (float)H, rC = 1.0f / (float)C;

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
                    const int r = div_small(e, rH);
                    sA[r * HS + (e - r * H)] = a[u];
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
                if (e < nW) {
                    const int r = div_small(e, rC);
                    sW[r * CP + (e - r * C)] = w[u];
                }
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
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar block/part arithmetic
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
            // four k-steps per batch: all of a batch's LDS reads go out before
            // its first MFMA.  Addresses are clamped in range and values past
            // the edges are multiplied by 0 rather than selected, so no read
            // is predicated (a predicated read waits before the next one is
            // issued); the zero steps past ke add exact zeros.
            const int bc = min(ba, rows - 1), cc = min(cb, C - 1);
            const float am = ba < rows ? 1.f : 0.f, wm = cb < C ? 1.f : 0.f;
            for (int k0 = kb; k0 < ke; k0 += 16) {
                float av[4], wv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + 4 * u + lk;
                    const int kc = min(k, ke - 1);
                    const float km = k < ke ? 1.f : 0.f;
                    av[u] = sA[bc * HS + kc] * (am * km);
                    wv[u] = sW[kc * CP + cc] * wm;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], wv[u], acc, 0, 0, 0);
            }
            s_red[wave][lane] = acc;
        }
        __syncthreads();
        if (wave < nb) {
            const int blk = wave;
            const int b0 = (blk / CB) * 16, c0 = (blk % CB) * 16;
            const int cb = c0 + li;
            // every part's sum is read before the adds (uniform predicate on
            // the count, clamped rows), then added in part order
            float4v zp[kHeadWaves];
#pragma unroll
            for (int part = 0; part < kHeadWaves; ++part) zp[part] = s_red[min(part * nb + blk, kHeadWaves - 1)][lane];
            float4v z = zp[0];
#pragma unroll
            for (int part = 1; part < kHeadWaves; ++part)
                if (part < KS) z += zp[part];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int bb = b0 + 4 * lk + e;
                if (bb < rows && cb < C) sZ[bb * C + cb] = z[e];
            }
        }
    }
    __syncthreads();

    // softmax cross-entropy, 16 lanes per row (classes j and j + 16 of the
    // row on lane j); max and sums across the 16-lane row by DPP moves in a
    // fixed order (row16_sum / row16_max).  Only LDS is written before the next barrier (a barrier
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
            const float mx = row16_max(fmaxf(z0, z1));
            const float e0 = v0 ? expf(z0 - mx) : 0.f, e1 = v1 ? expf(z1 - mx) : 0.f;
            const float se = row16_sum(e0 + e1);
            const float st = row16_sum(t0 + t1);
            const float stz = row16_sum((v0 ? t0 * z0 : 0.f) + (v1 ? t1 * z1 : 0.f));
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
        // K = C <= 32: every read of the block goes out before the MFMAs
        // (clamped addresses, edges multiplied by 0 as in the logits)
        const int bc = min(ba, rows - 1), hc = min(hb, H - 1);
        const float zm = ba < rows ? 1.f : 0.f, hm = hb < H ? 1.f : 0.f;
        float zv[8], wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int k = 4 * u + lk;
            const int kc = min(k, C - 1);
            const float km = k < C ? 1.f : 0.f;
            zv[u] = sZ[bc * C + kc] * (zm * km);
            wv[u] = sW[hc * CP + kc] * hm;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (4 * u < C) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(zv[u], wv[u], acc, 0, 0, 0);
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
