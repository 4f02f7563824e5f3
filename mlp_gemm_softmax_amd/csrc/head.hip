// Fused output layer for narrow class counts (C <= 32): one launch does the
// last matmul, the softmax cross-entropy, the dX of the last layer and its
// dW + SGD (README "Example": logits = matmul(h, w2) feeding
// cross_entropy_loss; the backward that autodiff derives for them).
//
// Each workgroup (16 waves) owns RB batch rows; W_L [H][C] and the rows'
// activations, labels and masks are staged in LDS.  Per workgroup:
//   logits[b][c] = sum_h a[b][h] W[h][c]                (fixed order)
//   lane-per-row softmax-CE -> dlogits, row loss         (as the CE kernel)
//   G[b][h] = mask[b][h] * sum_c dlogits[b][c] W[h][c]   (old W)
//   P_blk[h][c] = sum_{b in block} a[b][h] dlogits[b][c] (partial dW)
// The workgroup that draws the last integer ticket adds the partials in block
// order, applies W -= lr * dW (or stores dW) and averages the row losses in
// row order.  Every other workgroup has finished reading W before it takes
// its ticket, so the in-place update is safe.  For small batches this
// replaces five launches (logits GEMM, CE, dX GEMM, dW GEMM and the loss
// mean) whose run time is dominated by launch and memory latency.
#include <math.h>

#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void head_kernel(HeadParams p) {
    extern __shared__ float lds[];
    __shared__ int s_last;
    const int H = p.H, C = p.C, CP = p.CP, RB = p.RB;
    const int HS = H | 1;             // odd LDS row stride: rows land on distinct banks
    float* sW = lds;                  // [H][CP]
    float* sA = sW + H * CP;          // [RB][HS]
    float* sZ = sA + RB * HS;         // [RB][C]  logits, then dlogits
    float* sT = sZ + RB * C;          // [RB][C]  labels
    uint8_t* sM = (uint8_t*)(sT + RB * C);   // [RB][H] mask
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;
    const int row0 = blk * RB;
    const int rows = min(RB, p.B - row0);

    // Stage everything the block reads once, all loads in flight together.
    for (int e = tid; e < H * C; e += kThreads) sW[(e / C) * CP + e % C] = p.W[e];
    for (int e = tid; e < rows * H; e += kThreads) {
        sA[(e / H) * HS + e % H] = p.A[(int64_t)row0 * H + e];
        sM[e] = p.mask[(int64_t)row0 * H + e];
    }
    for (int e = tid; e < rows * C; e += kThreads) sT[e] = p.labels[(int64_t)row0 * C + e];
    __syncthreads();

    // logits; four interleaved partial sums (h mod 4) combined in fixed order
    for (int e = tid; e < rows * C; e += kThreads) {
        const int b = e / C, c = e % C;
        const float* a = sA + b * HS;
        const float* w = sW + c;
        float z0 = 0.f, z1 = 0.f, z2 = 0.f, z3 = 0.f;
        int h = 0;
#pragma unroll 4
        for (; h + 4 <= H; h += 4) {
            z0 += a[h] * w[h * CP];
            z1 += a[h + 1] * w[(h + 1) * CP];
            z2 += a[h + 2] * w[(h + 2) * CP];
            z3 += a[h + 3] * w[(h + 3) * CP];
        }
        for (; h < H; ++h) z0 += a[h] * w[h * CP];
        const float z = (z0 + z1) + (z2 + z3);
        sZ[b * C + c] = z;
        if (p.logits) p.logits[(int64_t)(row0 + b) * C + c] = z;
    }
    __syncthreads();

    // softmax cross-entropy, one lane per row
    if (tid < rows) {
        const int b = tid, row = row0 + b;
        const float* t = sT + b * C;
        float* z = sZ + b * C;
        float mx = -INFINITY;
        for (int c = 0; c < C; ++c) mx = fmaxf(mx, z[c]);
        float se = 0.f, st = 0.f, stz = 0.f;
        for (int c = 0; c < C; ++c) {
            const float tc = t[c];
            st += tc;
            stz += tc * z[c];
            se += expf(z[c] - mx);
        }
        const float lse = mx + logf(se);
        for (int c = 0; c < C; ++c) {
            const float g = (expf(z[c] - mx) / se * st - t[c]) * p.inv_b;
            z[c] = g;
            p.dlogits[(int64_t)row * C + c] = g;
        }
        store_coherent(p.rowloss + row, st * lse - stz);
    }
    __syncthreads();

    // dX of the last layer through the ReLU mask (four outputs per pass)
    for (int e0 = tid; e0 < rows * H; e0 += 4 * kThreads) {
        float g[4];
        int eo[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * kThreads;
            eo[u] = e;
            g[u] = 0.f;
            if (e < rows * H) {
                const float* z = sZ + (e / H) * C;
                const float* w = sW + (e % H) * CP;
                for (int c = 0; c < C; ++c) g[u] += z[c] * w[c];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (eo[u] < rows * H) {
                p.G[(int64_t)row0 * H + eo[u]] = sM[eo[u]] ? g[u] : 0.f;
            }
        }
    }

    // partial dW over this block's rows; four interleaved partial sums
    float* part = p.partials + (int64_t)blk * H * C;
    for (int e = tid; e < H * C; e += kThreads) {
        const int h = e / C, c = e % C;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        int b = 0;
#pragma unroll 4
        for (; b + 4 <= rows; b += 4) {
            s0 += sA[b * HS + h] * sZ[b * C + c];
            s1 += sA[(b + 1) * HS + h] * sZ[(b + 1) * C + c];
            s2 += sA[(b + 2) * HS + h] * sZ[(b + 2) * C + c];
            s3 += sA[(b + 3) * HS + h] * sZ[(b + 3) * C + c];
        }
        for (; b < rows; ++b) s0 += sA[b * HS + h] * sZ[b * C + c];
        store_coherent(part + e, (s0 + s1) + (s2 + s3));
    }

    if (!last_arrival(p.ticket, gridDim.x, &s_last)) return;

    // dW in block order, then the update (or the stored gradient).  The loads
    // of up to 8 blocks are issued before any is added, so the reduction costs
    // a few memory round trips rather than one per block.
    const int nblk = gridDim.x;
    for (int e = tid; e < H * C; e += kThreads) {
        float s = 0.f;
        for (int k0 = 0; k0 < nblk; k0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = k0 + u < nblk ? load_coherent(p.partials + (int64_t)(k0 + u) * H * C + e) : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        if (p.dW) p.dW[e] = s;
        else p.W[e] = sW[(e / C) * CP + e % C] - p.lr * s;
    }
    // mean loss in row order
    float s = 0.f;
    for (int b0 = tid; b0 < p.B; b0 += 4 * kThreads) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int b = b0 + u * kThreads;
            v[u] = b < p.B ? load_coherent(p.rowloss + b) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) s += v[u];
    }
    s = wave_sum(s);
    __shared__ float part_sum[kThreads / kWave];
    if ((tid & 63) == 0) part_sum[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int w = 0; w < kThreads / kWave; ++w) tot += part_sum[w];
        *p.loss = tot * p.inv_b;
    }
}

}  // namespace

size_t head_lds_bytes(int H, int C, int RB) {
    const int CP = C | 1, HS = H | 1;
    return sizeof(float) * ((size_t)H * CP + (size_t)RB * HS + 2 * (size_t)RB * C) + (size_t)RB * H;
}

int head_max_lds() { return 96 * 1024; }

hipError_t head_prepare() {
    return hipFuncSetAttribute((const void*)head_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               head_max_lds());
}

hipError_t launch_head(const HeadParams& p, hipStream_t s) {
    const int grid = (p.B + p.RB - 1) / p.RB;
    hipLaunchKernelGGL(head_kernel, dim3(grid), dim3(kThreads), head_lds_bytes(p.H, p.C, p.RB), s, p);
    return hipGetLastError();
}

}  // namespace mlp
