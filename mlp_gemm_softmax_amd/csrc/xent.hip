// Row-wise softmax cross-entropy against dense labels (the README's
// cross_entropy_loss(logits, labels), "Example" section) in one kernel: the
// reduction archetype.  Per row b
//   mu = max_c z,  S = sum_c exp(z - mu),  lse = mu + log S,
//   s = sum_c t,   loss_b = s*lse - sum_c t*z,
//   dlogits = (exp(z - mu)/S * s - t) / B.
// Narrow rows (C <= 32) take one lane per row, so a wavefront handles 64 rows
// and no cross-lane reduction is needed; wider rows take one wavefront per
// row, with max and sums by xor-butterfly shuffles across the 64 lanes.
// Mean loss: row losses are stored with device-scope stores, each workgroup
// takes an integer ticket, and the last one sums all B row losses in a fixed
// order (at most 256 workgroups draw tickets, bounding atomic contention).
#include <math.h>

#include <algorithm>

#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxGroups = 256;
// mean_rows_wave (the mean taken by the next launch in skinny steps) repeats
// finish_mean's additions for four wavefronts; both must change together.
static_assert(kThreads / kWave == 4, "finish_mean and mean_rows_wave add four wavefront sums");

__device__ void finish_mean(const XentParams& p) {
    // Last workgroup only: fixed-order sum of the row losses.
    const int tid = threadIdx.x;
    // loads of 8 rows in flight before they are added (row order kept)
    float s = 0.f;
    for (int b0 = tid; b0 < p.B; b0 += 8 * kThreads) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int b = b0 + u * kThreads;
            v[u] = b < p.B ? load_coherent(p.rowloss + b) : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    s = wave_sum(s);
    __shared__ float part[kThreads / kWave];
    if ((tid & 63) == 0) part[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int w = 0; w < kThreads / kWave; ++w) tot += part[w];
        *p.loss = tot * p.inv_b;
    }
}

// One lane per row, C <= CMAX.
template <int CMAX>
__global__ __launch_bounds__(kThreads) void xent_lane(XentParams p) {
    __shared__ int s_last;
    const int row = blockIdx.x * kThreads + threadIdx.x;
    if (row < p.B) {
        const float* z = p.logits + (int64_t)row * p.C;
        const float* t = p.labels + (int64_t)row * p.C;
        float zv[CMAX], tv[CMAX];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < CMAX; ++c) {
            const bool ok = c < p.C;
            zv[c] = ok ? z[c] : -INFINITY;
            tv[c] = ok ? t[c] : 0.f;
            mx = fmaxf(mx, zv[c]);
        }
        float se = 0.f, st = 0.f, stz = 0.f;
#pragma unroll
        for (int c = 0; c < CMAX; ++c) {
            if (c < p.C) {
                st += tv[c];
                stz += tv[c] * zv[c];
                zv[c] = expf(zv[c] - mx);
                se += zv[c];
            }
        }
        const float lse = mx + logf(se);
        float* d = p.dlogits + (int64_t)row * p.C;
        bf16_t* db = p.dlogits_b ? p.dlogits_b + (int64_t)row * p.C : nullptr;
#pragma unroll
        for (int c = 0; c < CMAX; ++c) {
            if (c < p.C) {
                const float g = (zv[c] / se * st - tv[c]) * p.inv_b;
                d[c] = g;
                if (db) db[c] = f32_to_bf16(g);
            }
        }
        store_coherent(p.rowloss + row, st * lse - stz);
    }
    if (!p.defer_mean && last_arrival(p.ticket, gridDim.x, &s_last)) finish_mean(p);
}

// One wavefront per row, whole row in registers (C <= 64 * VPT); rows are
// strided over the grid's wavefronts, and the next row's logits and labels
// are loaded (from a clamped in-range row, unconditionally) before the
// current row is reduced, so each wave pays one memory round trip rather
// than one per row.
template <int VPT>
__global__ __launch_bounds__(kThreads) void xent_wave(XentParams p) {
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * (kThreads / kWave);
    float zn[VPT], tn[VPT];
    auto fetch = [&](int row) {
        const float* z = p.logits + (int64_t)min(row, p.B - 1) * p.C;
        const float* t = p.labels + (int64_t)min(row, p.B - 1) * p.C;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = min(lane + kWave * i, p.C - 1);
            zn[i] = z[c];
            tn[i] = t[c];
        }
    };
    // wide rows (VPT > 16) are not double-buffered: the registers would spill
    constexpr bool kAhead = VPT <= 16;
    int row = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
    if (kAhead && row < p.B) fetch(row);
    for (; row < p.B; row += waves) {
        if (!kAhead) fetch(row);
        float zv[VPT], tv[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            zv[i] = zn[i];
            tv[i] = tn[i];
        }
        if (kAhead && row + waves < p.B) fetch(row + waves);
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const bool ok = lane + kWave * i < p.C;
            zv[i] = ok ? zv[i] : -INFINITY;
            tv[i] = ok ? tv[i] : 0.f;
            mx = fmaxf(mx, zv[i]);
        }
        mx = wave_max(mx);
        float se = 0.f, st = 0.f, stz = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = lane + kWave * i;
            if (c < p.C) {
                st += tv[i];
                stz += tv[i] * zv[i];
                zv[i] = expf(zv[i] - mx);
                se += zv[i];
            }
        }
        se = wave_sum(se);
        st = wave_sum(st);
        stz = wave_sum(stz);
        const float lse = mx + logf(se);
        float* d = p.dlogits + (int64_t)row * p.C;
        bf16_t* db = p.dlogits_b ? p.dlogits_b + (int64_t)row * p.C : nullptr;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = lane + kWave * i;
            if (c < p.C) {
                const float g = (zv[i] / se * st - tv[i]) * p.inv_b;
                d[c] = g;
                if (db) db[c] = f32_to_bf16(g);
            }
        }
        if (lane == 0) store_coherent(p.rowloss + row, st * lse - stz);
    }
    if (!p.defer_mean && last_arrival(p.ticket, gridDim.x, &s_last)) finish_mean(p);
}

// Split-K sum and softmax-CE in one pass, for an output layer whose logits
// product was split over K: the partial sums [split][B][C] are added in split
// order (the order of the split-K epilogue, so the logits are the same), the
// logits are stored, and the row's loss and dlogits follow as in xent_wave.
// One wavefront per row, lane l holding float4 columns 4(l + 64 i); the next
// row's partials and labels are loaded before the current row is reduced.
// C is a multiple of 4 and at most 256 * V4 <= 1024.
constexpr int kMaxSplitsXent = 4;

template <int V4>
__global__ __launch_bounds__(kThreads) void splitk_xent_kernel(XentParams p, const float* __restrict__ partials,
                                                                 int splits, float* __restrict__ logits) {
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * (kThreads / kWave);
    const int64_t bc = (int64_t)p.B * p.C;
    float4v zn[kMaxSplitsXent][V4], tn[V4];
    auto fetch = [&](int row) {
        const int64_t base = (int64_t)min(row, p.B - 1) * p.C;
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int c = min(4 * (lane + kWave * i), p.C - 4);
#pragma unroll
            for (int t = 0; t < kMaxSplitsXent; ++t)   // splits past the last re-read it
                zn[t][i] = *reinterpret_cast<const float4v*>(partials + min(t, splits - 1) * bc + base + c);
            tn[i] = *reinterpret_cast<const float4v*>(p.labels + base + c);
        }
    };
    int row = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6);
    if (row < p.B) fetch(row);
    for (; row < p.B; row += waves) {
        float4v zv[V4], tv[V4];
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            zv[i] = zn[0][i];
#pragma unroll
            for (int t = 1; t < kMaxSplitsXent; ++t)
                if (t < splits) zv[i] += zn[t][i];
            tv[i] = tn[i];
        }
        if (row + waves < p.B) fetch(row + waves);
        const int64_t base = (int64_t)row * p.C;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int c = 4 * (lane + kWave * i);
            if (c < p.C) {
                *reinterpret_cast<float4v*>(logits + base + c) = zv[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) mx = fmaxf(mx, zv[i][e]);
            }
        }
        mx = wave_max(mx);
        float se = 0.f, st = 0.f, stz = 0.f;
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            if (4 * (lane + kWave * i) < p.C) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    st += tv[i][e];
                    stz += tv[i][e] * zv[i][e];
                    zv[i][e] = expf(zv[i][e] - mx);
                    se += zv[i][e];
                }
            }
        }
        se = wave_sum(se);
        st = wave_sum(st);
        stz = wave_sum(stz);
        const float lse = mx + logf(se);
#pragma unroll
        for (int i = 0; i < V4; ++i) {
            const int c = 4 * (lane + kWave * i);
            if (c < p.C) {
                float4v g;
#pragma unroll
                for (int e = 0; e < 4; ++e) g[e] = (zv[i][e] / se * st - tv[i][e]) * p.inv_b;
                *reinterpret_cast<float4v*>(p.dlogits + base + c) = g;
                if (p.dlogits_b) {
                    uint2 h;
                    h.x = pack2_bf16(g[0], g[1]);
                    h.y = pack2_bf16(g[2], g[3]);
                    *reinterpret_cast<uint2*>(p.dlogits_b + base + c) = h;
                }
            }
        }
        if (lane == 0) store_coherent(p.rowloss + row, st * lse - stz);
    }
    if (!p.defer_mean && last_arrival(p.ticket, gridDim.x, &s_last)) finish_mean(p);
}

// One workgroup per row, for few wide rows (B small, C large): the row is
// spread over 256 lanes (VPT values each); max and sums go through the
// wavefront butterflies and then LDS in wave order.
template <int VPT>
__global__ __launch_bounds__(kThreads) void xent_group(XentParams p) {
    __shared__ int s_last;
    __shared__ float red[3][kThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    const float* z = p.logits + (int64_t)row * p.C;
    const float* t = p.labels + (int64_t)row * p.C;
    float zv[VPT], tv[VPT];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = tid + kThreads * i;
        const bool ok = c < p.C;
        zv[i] = ok ? z[c] : -INFINITY;
        tv[i] = ok ? t[c] : 0.f;
        mx = fmaxf(mx, zv[i]);
    }
    mx = wave_max(mx);
    if (lane == 0) red[0][wave] = mx;
    __syncthreads();
    mx = red[0][0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) mx = fmaxf(mx, red[0][w]);
    float se = 0.f, st = 0.f, stz = 0.f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = tid + kThreads * i;
        if (c < p.C) {
            st += tv[i];
            stz += tv[i] * zv[i];
            zv[i] = expf(zv[i] - mx);
            se += zv[i];
        }
    }
    se = wave_sum(se);
    st = wave_sum(st);
    stz = wave_sum(stz);
    __syncthreads();
    if (lane == 0) {
        red[0][wave] = se;
        red[1][wave] = st;
        red[2][wave] = stz;
    }
    __syncthreads();
    se = red[0][0];
    st = red[1][0];
    stz = red[2][0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) {
        se += red[0][w];
        st += red[1][w];
        stz += red[2][w];
    }
    const float lse = mx + logf(se);
    float* d = p.dlogits + (int64_t)row * p.C;
    bf16_t* db = p.dlogits_b ? p.dlogits_b + (int64_t)row * p.C : nullptr;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = tid + kThreads * i;
        if (c < p.C) {
            const float g = (zv[i] / se * st - tv[i]) * p.inv_b;
            d[c] = g;
            if (db) db[c] = f32_to_bf16(g);
        }
    }
    if (tid == 0) store_coherent(p.rowloss + row, st * lse - stz);
    if (!p.defer_mean && last_arrival(p.ticket, gridDim.x, &s_last)) finish_mean(p);
}

// Any C: running (max, sum) per lane in one sweep, merged across lanes, then
// a second sweep writes dlogits.
__global__ __launch_bounds__(kThreads) void xent_stream(XentParams p) {
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int waves = gridDim.x * (kThreads / kWave);
    for (int row = blockIdx.x * (kThreads / kWave) + (threadIdx.x >> 6); row < p.B; row += waves) {
        const float* z = p.logits + (int64_t)row * p.C;
        const float* t = p.labels + (int64_t)row * p.C;
        float m = -INFINITY, se = 0.f, st = 0.f, stz = 0.f;
        for (int c = lane; c < p.C; c += kWave) {
            const float zc = z[c], tc = t[c];
            if (zc > m) {
                se = se * expf(m - zc) + 1.f;
                m = zc;
            } else {
                se += expf(zc - m);
            }
            st += tc;
            stz += tc * zc;
        }
        const float mx = wave_max(m);
        se = wave_sum(m == -INFINITY ? 0.f : se * expf(m - mx));
        st = wave_sum(st);
        stz = wave_sum(stz);
        const float lse = mx + logf(se);
        float* d = p.dlogits + (int64_t)row * p.C;
        bf16_t* db = p.dlogits_b ? p.dlogits_b + (int64_t)row * p.C : nullptr;
        for (int c = lane; c < p.C; c += kWave) {
            const float g = (expf(z[c] - mx) / se * st - t[c]) * p.inv_b;
            d[c] = g;
            if (db) db[c] = f32_to_bf16(g);
        }
        if (lane == 0) store_coherent(p.rowloss + row, st * lse - stz);
    }
    if (!p.defer_mean && last_arrival(p.ticket, gridDim.x, &s_last)) finish_mean(p);
}

// Class probabilities of each row (inference): the same normalisation as the
// loss, p = exp(z - mu) / S.  Each thread keeps its VPT values of the row in
// registers (every load in flight at once), so the row is read once:
// rows of up to 64 * VPT classes take one wavefront each, wider rows (up to
// kThreads * VPT) one workgroup each, with the four wavefronts' partial max
// and sum combined through LDS in wave order.  Still wider rows stream the
// row three times (max, sum, write).
template <int VPT, bool GROUP>
__global__ __launch_bounds__(kThreads) void softmax_rows(const float* __restrict__ logits,
                                                         float* __restrict__ probs, int B, int C) {
    __shared__ float s_red[2][kThreads / kWave];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int kWaves = kThreads / kWave;
    const int width = GROUP ? kThreads : kWave;           // threads per row
    const int t = GROUP ? (int)threadIdx.x : lane;
    const int rows_per_group = GROUP ? 1 : kWaves;
    for (int row = blockIdx.x * rows_per_group + (GROUP ? 0 : wave); row < B; row += gridDim.x * rows_per_group) {
        const float* z = logits + (int64_t)row * C;
        float v[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = t + i * width;
            v[i] = c < C ? z[c] : -INFINITY;
        }
        float mx = v[0];
#pragma unroll
        for (int i = 1; i < VPT; ++i) mx = fmaxf(mx, v[i]);
        mx = wave_max(mx);
        if constexpr (GROUP) {
            if (lane == 0) s_red[0][wave] = mx;
            __syncthreads();
            mx = s_red[0][0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, s_red[0][w]);
        }
        float se = 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            v[i] = t + i * width < C ? expf(v[i] - mx) : 0.f;
            se += v[i];
        }
        se = wave_sum(se);
        if constexpr (GROUP) {
            if (lane == 0) s_red[1][wave] = se;
            __syncthreads();
            se = s_red[1][0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) se += s_red[1][w];
            __syncthreads();   // s_red is reused by the next row
        }
        float* p = probs + (int64_t)row * C;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = t + i * width;
            if (c < C) p[c] = v[i] / se;
        }
    }
}

__global__ __launch_bounds__(kThreads) void softmax_rows_stream(const float* __restrict__ logits,
                                                                float* __restrict__ probs, int B, int C) {
    const int lane = threadIdx.x & 63;
    const int rows_per_group = kThreads / kWave;
    for (int row = blockIdx.x * rows_per_group + (threadIdx.x >> 6); row < B; row += gridDim.x * rows_per_group) {
        const float* z = logits + (int64_t)row * C;
        float mx = -INFINITY;
        for (int c = lane; c < C; c += kWave) mx = fmaxf(mx, z[c]);
        mx = wave_max(mx);
        float se = 0.f;
        for (int c = lane; c < C; c += kWave) se += expf(z[c] - mx);
        se = wave_sum(se);
        float* p = probs + (int64_t)row * C;
        for (int c = lane; c < C; c += kWave) p[c] = expf(z[c] - mx) / se;
    }
}

}  // namespace

hipError_t launch_softmax_rows(const float* logits, float* probs, int B, int C, hipStream_t st) {
    if (B < 1 || C < 1 || !logits || !probs) return hipErrorInvalidValue;
    const int rows_per_group = kThreads / kWave;
    const int wave_grid = std::min((B + rows_per_group - 1) / rows_per_group, 4 * kMaxGroups);
    const int group_grid = std::min(B, 4 * kMaxGroups);
#define MLP_SOFTMAX(V, G, GRID) hipLaunchKernelGGL((softmax_rows<V, G>), dim3(GRID), dim3(kThreads), 0, st, logits, probs, B, C)
    // wide rows with few of them: a workgroup per row keeps the CUs busy
    const bool group = C > 16 * kWave || (B < 512 && C > 4 * kWave);
    if (!group) {
        if (C <= kWave) MLP_SOFTMAX(1, false, wave_grid);
        else if (C <= 4 * kWave) MLP_SOFTMAX(4, false, wave_grid);
        else MLP_SOFTMAX(16, false, wave_grid);
    } else if (C <= 8 * kThreads) {
        MLP_SOFTMAX(8, true, group_grid);
    } else if (C <= 32 * kThreads) {
        MLP_SOFTMAX(32, true, group_grid);
    } else {
        hipLaunchKernelGGL(softmax_rows_stream, dim3(wave_grid), dim3(kThreads), 0, st, logits, probs, B, C);
    }
#undef MLP_SOFTMAX
    return hipGetLastError();
}

hipError_t launch_xent(const XentParams& p, int* grid_out, hipStream_t s) {
    int grid;
    if (p.C <= 32) {
        grid = (p.B + kThreads - 1) / kThreads;
        if (p.C <= 8) hipLaunchKernelGGL(xent_lane<8>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (p.C <= 16) hipLaunchKernelGGL(xent_lane<16>, dim3(grid), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL(xent_lane<32>, dim3(grid), dim3(kThreads), 0, s, p);
    } else if (p.B <= 64 && p.C >= 512 && p.C <= 32 * kThreads) {
        grid = p.B;
        const int vpt = (p.C + kThreads - 1) / kThreads;
        if (vpt <= 4) hipLaunchKernelGGL(xent_group<4>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 8) hipLaunchKernelGGL(xent_group<8>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 16) hipLaunchKernelGGL(xent_group<16>, dim3(grid), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL(xent_group<32>, dim3(grid), dim3(kThreads), 0, s, p);
    } else {
        const int rows_per_group = kThreads / kWave;
        grid = (p.B + rows_per_group - 1) / rows_per_group;
        if (grid > kMaxGroups) grid = kMaxGroups;
        const int vpt = (p.C + kWave - 1) / kWave;
        if (vpt <= 1) hipLaunchKernelGGL(xent_wave<1>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 2) hipLaunchKernelGGL(xent_wave<2>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 4) hipLaunchKernelGGL(xent_wave<4>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 8) hipLaunchKernelGGL(xent_wave<8>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 16) hipLaunchKernelGGL(xent_wave<16>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 32) hipLaunchKernelGGL(xent_wave<32>, dim3(grid), dim3(kThreads), 0, s, p);
        else if (vpt <= 64) hipLaunchKernelGGL(xent_wave<64>, dim3(grid), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL(xent_stream, dim3(grid), dim3(kThreads), 0, s, p);
    }
    if (grid_out) *grid_out = grid;
    return hipGetLastError();
}

bool splitk_xent_fits(int C, int splits) {
    return C >= 4 && C % 4 == 0 && C <= 256 * 4 && splits >= 2 && splits <= kMaxSplitsXent;
}

hipError_t launch_splitk_xent(const XentParams& p, const float* partials, int splits, float* logits,
                              hipStream_t s) {
    if (!splitk_xent_fits(p.C, splits) || p.B < 1 || !partials || !logits) return hipErrorInvalidValue;
    const int rows_per_group = kThreads / kWave;
    const int grid = std::min((p.B + rows_per_group - 1) / rows_per_group, 2 * kMaxGroups);
    const int v4 = (p.C + 4 * kWave - 1) / (4 * kWave);
    if (v4 <= 1) hipLaunchKernelGGL(splitk_xent_kernel<1>, dim3(grid), dim3(kThreads), 0, s, p, partials, splits, logits);
    else if (v4 <= 2) hipLaunchKernelGGL(splitk_xent_kernel<2>, dim3(grid), dim3(kThreads), 0, s, p, partials, splits, logits);
    else hipLaunchKernelGGL(splitk_xent_kernel<4>, dim3(grid), dim3(kThreads), 0, s, p, partials, splits, logits);
    return hipGetLastError();
}

}  // namespace mlp
