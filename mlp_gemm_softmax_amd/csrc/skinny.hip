// Skinny-batch (B <= 16) float32 kernels.  With a handful of rows every
// product of the step is a pass over a weight matrix, so these kernels are
// shaped for HBM streaming rather than for the matrix cores' peak:
//
//   skinny_nn  out[b][n] = sum_k x[b][k] W[k][n]          forward, W row-streamed
//   skinny_nt  out[b][k] = mask[b][k] * sum_n G[b][n] W[k][n]   dX (MFMA 16x16x4)
//   skinny_tn  W[k][n]  -= lr * sum_b a[b][k] G[b][n]     dW + SGD, one read+write of W
//
// All reductions have a fixed order: k-splits inside a workgroup are summed
// through LDS in wave order, splits across workgroups through partial buffers
// that the last workgroup (integer ticket) adds up in split order.
// Requires every width and K to be a multiple of 4 (float4 rows).
#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kCols = 4 * kWave;   // columns per wave in the row-streaming kernels

// ---------------------------------------------------------------------------
// Forward: each lane owns 4 consecutive output columns for all batch rows;
// the waves of a workgroup take interleaved groups of 4 rows of W from the
// workgroup's K chunk; grid = column blocks x K splits.
template <int MB, int NW, Epi EPI>
__global__ __launch_bounds__(NW * kWave) void skinny_nn(SkinnyParams p) {
    extern __shared__ float4 red[];   // [NW-1][MB][kWave] partial columns
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ncb = (p.N + kCols - 1) / kCols;
    const int id = blockIdx.x;
    const int cb = id % ncb, split = id / ncb;
    const int n = cb * kCols + 4 * lane;
    const bool nok = n < p.N;
    const int kbeg = split * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);

    float4 acc[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[b] = make_float4(0.f, 0.f, 0.f, 0.f);

    const float* __restrict__ W = p.B;
    const float* __restrict__ X = p.A;
    for (int k = kbeg + 4 * wave; k < kend; k += 4 * NW) {
        float4 w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            w[r] = nok ? *reinterpret_cast<const float4*>(W + (int64_t)(k + r) * p.N + n)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            if (b < p.MB) {
                const float4 xv = *reinterpret_cast<const float4*>(X + (int64_t)b * p.K + k);
                acc[b].x += xv.x * w[0].x; acc[b].y += xv.x * w[0].y;
                acc[b].z += xv.x * w[0].z; acc[b].w += xv.x * w[0].w;
                acc[b].x += xv.y * w[1].x; acc[b].y += xv.y * w[1].y;
                acc[b].z += xv.y * w[1].z; acc[b].w += xv.y * w[1].w;
                acc[b].x += xv.z * w[2].x; acc[b].y += xv.z * w[2].y;
                acc[b].z += xv.z * w[2].z; acc[b].w += xv.z * w[2].w;
                acc[b].x += xv.w * w[3].x; acc[b].y += xv.w * w[3].y;
                acc[b].z += xv.w * w[3].z; acc[b].w += xv.w * w[3].w;
            }
        }
    }

    // Sum the waves' partial columns in wave order 0..NW-1.
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < MB; ++b) red[((wave - 1) * MB + b) * kWave + lane] = acc[b];
    }
    __syncthreads();
    if (wave == 0) {
        for (int w = 1; w < NW; ++w)
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const float4 o = red[((w - 1) * MB + b) * kWave + lane];
                acc[b].x += o.x; acc[b].y += o.y; acc[b].z += o.z; acc[b].w += o.w;
            }
    }

    if (p.splits > 1) {
        if (wave == 0 && nok) {
#pragma unroll
            for (int b = 0; b < MB; ++b)
                if (b < p.MB)
                    *reinterpret_cast<float4*>(p.partials + ((int64_t)split * p.MB + b) * p.N + n) = acc[b];
        }
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned old = atomicAdd(&p.tickets[cb], 1u);
            const int last = old == (unsigned)(p.splits - 1);
            if (last) atomicExch(&p.tickets[cb], 0u);
            s_last = last;
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        // acquire done; add the splits in order t = 0..S-1
        if (wave == 0 && nok) {
            float4 sum[MB];
#pragma unroll
            for (int b = 0; b < MB; ++b) sum[b] = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int t = 0; t < p.splits; ++t) {
#pragma unroll
                for (int b = 0; b < MB; ++b) {
                    if (b < p.MB) {
                        const float4 o = t == split ? acc[b]
                            : *reinterpret_cast<const float4*>(p.partials + ((int64_t)t * p.MB + b) * p.N + n);
                        sum[b].x += o.x; sum[b].y += o.y; sum[b].z += o.z; sum[b].w += o.w;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < MB; ++b) acc[b] = sum[b];
        }
    }

    if (wave == 0 && nok) {
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            if (b >= p.MB) break;
            float4 v = acc[b];
            const int64_t o = (int64_t)b * p.N + n;
            if constexpr (EPI == Epi::ReluMask) {
                uchar4 m;
                m.x = v.x > 0.f; m.y = v.y > 0.f; m.z = v.z > 0.f; m.w = v.w > 0.f;
                v.x = m.x ? v.x : 0.f; v.y = m.y ? v.y : 0.f;
                v.z = m.z ? v.z : 0.f; v.w = m.w ? v.w : 0.f;
                *reinterpret_cast<uchar4*>(p.mask + o) = m;
            }
            *reinterpret_cast<float4*>(p.C + o) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// dX: out[b][k] = mask[b][k] * sum_n G[b][n] W[k][n], W stored [Kout][N].
// v_mfma_f32_16x16x4f32 with A = 16 rows of W and B = G^T (16 batch columns,
// the ones >= B zero): lane l supplies W[k0 + l%16][n + 4(l/16) + q] and
// G[l%16][n + 4(l/16) + q] to MFMA q, so one float4 of each feeds four MFMAs
// and the reduction over n happens inside the matrix core.  A workgroup of
// 4 waves covers 16 rows of W; wave w takes the w-th quarter of n.
__global__ __launch_bounds__(256) void skinny_nt(SkinnyParams p) {
    __shared__ float4 red[3][kWave];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int k0 = blockIdx.x * 16;
    const int i = lane & 15, g = lane >> 4;
    const int krow = k0 + i;
    const bool rok = krow < p.K;
    const bool bok = i < p.MB;
    // quarter of the n range, in multiples of 16
    const int nq = ((p.N + 63) / 64) * 16;
    const int nbeg = wave * nq;
    const int nend = min(p.N, nbeg + nq);

    float4v acc = {0.f, 0.f, 0.f, 0.f};
    const float* __restrict__ Wr = p.A + (int64_t)krow * p.N;
    const float* __restrict__ Gr = p.B + (int64_t)i * p.N;
    for (int n = nbeg; n < nend; n += 16) {
        const int c = n + 4 * g;
        float4v w = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
        if (c < nend) {
            if (rok) w = *reinterpret_cast<const float4v*>(Wr + c);
            if (bok) gv = *reinterpret_cast<const float4v*>(Gr + c);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(w[q], gv[q], acc, 0, 0, 0);
    }
    if (wave > 0) red[wave - 1][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < 3; ++w) {
        const float4 o = red[w][lane];
        acc[0] += o.x; acc[1] += o.y; acc[2] += o.z; acc[3] += o.w;
    }
    // acc[r] = out[b = lane%16][k = k0 + 4*(lane/16) + r]
    const int b = lane & 15;
    const int k = k0 + 4 * (lane >> 4);
    if (b < p.MB && k < p.K) {
        const int64_t o = (int64_t)b * p.K + k;
        float4 v = make_float4(acc[0], acc[1], acc[2], acc[3]);
        if (p.mask) {
            const uchar4 m = *reinterpret_cast<const uchar4*>(p.mask + o);
            v.x = m.x ? v.x : 0.f; v.y = m.y ? v.y : 0.f;
            v.z = m.z ? v.z : 0.f; v.w = m.w ? v.w : 0.f;
        }
        *reinterpret_cast<float4*>(p.C + o) = v;
    }
}

// ---------------------------------------------------------------------------
// dW + SGD: W[k][n] -= lr * sum_b a[b][k] G[b][n] (or store the gradient).
// Each lane keeps G[0..B)[n..n+3] in registers and walks ROWS rows of W, so W
// is read once and written once.  The per-row a[b][k] are staged in LDS.
template <int MB, int ROWS, Epi EPI>
__global__ __launch_bounds__(256) void skinny_tn(SkinnyParams p) {
    __shared__ float sa[ROWS][MB];
    const int ncb = (p.N + 4 * 256 - 1) / (4 * 256);
    const int cb = blockIdx.x % ncb, rb = blockIdx.x / ncb;
    const int k0 = rb * ROWS;
    const int n = cb * 1024 + 4 * threadIdx.x;
    for (int e = threadIdx.x; e < ROWS * MB; e += 256) {
        const int r = e / MB, b = e % MB;
        sa[r][b] = (b < p.MB && k0 + r < p.K) ? p.A[(int64_t)b * p.K + k0 + r] : 0.f;
    }
    __syncthreads();
    if (n >= p.N) return;
    float4 gv[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
        gv[b] = b < p.MB ? *reinterpret_cast<const float4*>(p.B + (int64_t)b * p.N + n)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    const int rows = min(ROWS, p.K - k0);
    float4 w[ROWS];
    if constexpr (EPI == Epi::Sgd) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            if (r < rows) w[r] = *reinterpret_cast<const float4*>(p.C + (int64_t)(k0 + r) * p.N + n);
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        if (r >= rows) break;
        float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            const float a = sa[r][b];
            d.x += a * gv[b].x; d.y += a * gv[b].y; d.z += a * gv[b].z; d.w += a * gv[b].w;
        }
        const int64_t o = (int64_t)(k0 + r) * p.N + n;
        if constexpr (EPI == Epi::Sgd) {
            float4 v = w[r];
            v.x -= p.lr * d.x; v.y -= p.lr * d.y; v.z -= p.lr * d.z; v.w -= p.lr * d.w;
            *reinterpret_cast<float4*>(p.C + o) = v;
        } else {
            *reinterpret_cast<float4*>(p.C + o) = d;
        }
    }
}

template <int MB>
hipError_t go_mb(const SkinnyLaunch& L, const SkinnyParams& p, hipStream_t s) {
    switch (L.layout) {
    case Layout::NN: {
        const size_t lds = (size_t)(L.waves - 1) * MB * kWave * sizeof(float4);
#define MLP_NN(NWV)                                                                              \
    if (L.waves == NWV) {                                                                        \
        if (L.epi == Epi::ReluMask)                                                              \
            hipLaunchKernelGGL((skinny_nn<MB, NWV, Epi::ReluMask>), dim3(L.grid), dim3(NWV * 64), \
                               lds, s, p);                                                       \
        else                                                                                     \
            hipLaunchKernelGGL((skinny_nn<MB, NWV, Epi::Store>), dim3(L.grid), dim3(NWV * 64),    \
                               lds, s, p);                                                       \
        return hipGetLastError();                                                                \
    }
        MLP_NN(4)
        MLP_NN(8)
#undef MLP_NN
        return hipErrorInvalidValue;
    }
    case Layout::NT:
        hipLaunchKernelGGL(skinny_nt, dim3(L.grid), dim3(256), 0, s, p);
        return hipGetLastError();
    case Layout::TN:
        if (L.epi == Epi::Sgd)
            hipLaunchKernelGGL((skinny_tn<MB, 16, Epi::Sgd>), dim3(L.grid), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((skinny_tn<MB, 16, Epi::Grad>), dim3(L.grid), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_skinny(const SkinnyLaunch& L, const SkinnyParams& p, hipStream_t s) {
    if (p.MB <= 2) return go_mb<2>(L, p, s);
    if (p.MB <= 4) return go_mb<4>(L, p, s);
    if (p.MB <= 8) return go_mb<8>(L, p, s);
    if (p.MB <= 16) return go_mb<16>(L, p, s);
    return hipErrorInvalidValue;
}

}  // namespace mlp
