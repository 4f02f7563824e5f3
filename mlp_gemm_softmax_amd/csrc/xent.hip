// Row-wise softmax cross-entropy against dense labels (the README's
// cross_entropy_loss(logits, labels), "Example" section) in one kernel: the
// reduction archetype.  One wavefront per row; per row b
//   mu = max_c z,  S = sum_c exp(z - mu),  lse = mu + log S,
//   s = sum_c t,   loss_b = s*lse - sum_c t*z,
//   dlogits = (exp(z - mu)/S * s - t) / B,
// with max and sums taken by xor-butterfly shuffles across the 64 lanes.
// Mean loss: every workgroup stores its rows' losses, takes an integer ticket,
// and the last workgroup sums all B row losses in a fixed order.
#include <math.h>

#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kRows = 4;           // rows (wavefronts) per workgroup
constexpr int kThreads = kRows * kWave;

__device__ void finish_mean(const XentParams& p) {
    // Called by the last workgroup only: fixed-order sum of row losses.
    const int tid = threadIdx.x;
    float s = 0.f;
    for (int b = tid; b < p.B; b += kThreads) s += p.rowloss[b];
    s = wave_sum(s);
    __shared__ float part[kRows];
    if ((tid & 63) == 0) part[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int w = 0; w < kRows; ++w) tot += part[w];
        *p.loss = tot * p.inv_b;
    }
}

__device__ void take_ticket_and_finish(const XentParams& p) {
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = atomicAdd(p.ticket, 1u);
        const int last = old == gridDim.x - 1;
        if (last) atomicExch(p.ticket, 0u);
        s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    finish_mean(p);
}

// Whole row in registers: C <= 64 * VPT.  Reads logits and labels once.
template <int VPT>
__global__ __launch_bounds__(kThreads) void xent_regs(XentParams p) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kRows + (threadIdx.x >> 6);
    if (row < p.B) {
        const float* z = p.logits + (int64_t)row * p.C;
        const float* t = p.labels + (int64_t)row * p.C;
        float zv[VPT], tv[VPT];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = lane + kWave * i;
            const bool ok = c < p.C;
            zv[i] = ok ? z[c] : -INFINITY;
            tv[i] = ok ? t[c] : 0.f;
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
        if (lane == 0) p.rowloss[row] = st * lse - stz;
    }
    take_ticket_and_finish(p);
}

// Any C: running (max, sum) per lane in one sweep, merged across lanes, then
// a second sweep writes dlogits.
__global__ __launch_bounds__(kThreads) void xent_stream(XentParams p) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kRows + (threadIdx.x >> 6);
    if (row < p.B) {
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
        if (lane == 0) p.rowloss[row] = st * lse - stz;
    }
    take_ticket_and_finish(p);
}

}  // namespace

hipError_t launch_xent(const XentParams& p, int* grid_out, hipStream_t s) {
    const int grid = (p.B + kRows - 1) / kRows;
    if (grid_out) *grid_out = grid;
    const int vpt = (p.C + kWave - 1) / kWave;
    if (vpt <= 1) hipLaunchKernelGGL(xent_regs<1>, dim3(grid), dim3(kThreads), 0, s, p);
    else if (vpt <= 2) hipLaunchKernelGGL(xent_regs<2>, dim3(grid), dim3(kThreads), 0, s, p);
    else if (vpt <= 4) hipLaunchKernelGGL(xent_regs<4>, dim3(grid), dim3(kThreads), 0, s, p);
    else if (vpt <= 8) hipLaunchKernelGGL(xent_regs<8>, dim3(grid), dim3(kThreads), 0, s, p);
    else if (vpt <= 16) hipLaunchKernelGGL(xent_regs<16>, dim3(grid), dim3(kThreads), 0, s, p);
    else if (vpt <= 32) hipLaunchKernelGGL(xent_regs<32>, dim3(grid), dim3(kThreads), 0, s, p);
    else if (vpt <= 64) hipLaunchKernelGGL(xent_regs<64>, dim3(grid), dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(xent_stream, dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mlp
