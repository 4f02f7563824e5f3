// Skinny-batch (B <= 16) float32 kernels.  With a handful of rows every
// product of the step is one pass over a weight matrix, so these kernels are
// shaped for HBM streaming rather than for the matrix cores' peak:
//
//   skinny_nn  out[b][n] = sum_k x[b][k] W[k][n]               forward
//   skinny_ntu out[b][k] = mask[b][k] * sum_n G[b][n] W[k][n]   dX, and
//              W[k][n] -= lr * sum_b a[b][k] G[b][n]           its dW + SGD,
//              in one pass over W (hidden layers)
//   skinny_tn  W[k][n]  -= lr * sum_b a[b][k] G[b][n]          dW + SGD (first layer)
//   skinny_nn with MBT > 0: the first layer's dW + SGD of one step and the
//              next step's forward of that layer, in one pass over W
//
// skinny_nn and skinny_ntu reduce inside v_mfma_f32_16x16x4f32 (the batch is
// the MFMA's 16-wide M or N side, rows >= B are zero), so every 16-byte load
// of W feeds four MFMAs and no cross-lane reduction is spent on K.  skinny_tn
// is a rank-B update streamed row by row: W is read once and written once.
// All reductions have a fixed order: the waves of a workgroup meet in LDS in
// wave order, and K splits across workgroups go through partial buffers that
// the last workgroup (integer ticket) adds in split order.
// Every width and K must be a multiple of 4 (float4 rows).
#include "kernels.hpp"
#include "optim_rule.hpp"

namespace mlp {
namespace {

__device__ __forceinline__ float4v ld4(const float* p) { return *reinterpret_cast<const float4v*>(p); }

// ---------------------------------------------------------------------------
// Forward.  A workgroup of NW waves owns 64 output columns n0..n0+63 and one
// K chunk; wave w takes the w-th contiguous slice of the chunk, 16 rows at a
// time.  Inside a 16-row block starting at k, MFMA step i (0..3) and k-lane
// group g (0..3) stand for row k + 4g + i, so lane (j = lane%16, g) loads
// W[k+4g+i][n0+4j .. n0+4j+3] for step i, and x[m = lane%16][k+4g .. k+4g+3]
// once for the block.  MFMA q (0..3) of step i multiplies component q of the
// W row: output column n0 + 4j + q.
//
// With MBT > 0 (batch rows padded to MBT = 4 or 8) the launch also finishes
// the previous step's first layer: every element of W it loads is updated,
// W' = W - lr * sum_b a[b][k] G[b][n] with the previous step's input a
// (p.act) and gradient G (p.grad), in exactly the arithmetic of skinny_tn
// (b ascending, one fma per b, then one fma for the step), stored once by the
// lane that loaded it (p.wout, in place), and W' is what this forward
// multiplies.  Results are bitwise those of skinny_tn followed by the plain
// forward on the next batch.
template <int NW, Epi EPI, int MBT = 0>
__global__ __launch_bounds__(NW * kWave) void skinny_nn(SkinnyParams p) {
    constexpr bool UPD = MBT > 0;
    __shared__ float4v red[NW - 1][4][kWave];
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, g = lane >> 4;
    const int ncg = (p.N + 63) / 64;
    const int cg = blockIdx.x % ncg, split = blockIdx.x / ncg;
    const int n = cg * 64 + 4 * j;
    const bool nok = n < p.N;
    const bool mok = j < p.MB;
    const int kbeg = split * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    // this wave's slice of the chunk, in whole 16-row blocks
    const int blocks = (kend - kbeg + 15) / 16;
    const int per = (blocks + NW - 1) / NW;
    const int kw0 = kbeg + wave * per * 16;
    const int kw1 = min(kend, kw0 + per * 16);

    float4v acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = {0.f, 0.f, 0.f, 0.f};

    // Loads are branch-free: lanes past N or past the slice read a valid
    // address (the matrix base) and zero the value.  The next block's loads
    // are issued before the current block's MFMAs, so memory latency overlaps
    // the matrix-core work.
    // (not __restrict__: with MBT > 0 the same rows are written through p.wout)
    const float* W = p.B;
    const float* __restrict__ X = p.A + (int64_t)(mok ? j : 0) * p.K;
    // One block is in flight ahead of the one being multiplied in the plain
    // forward (deeper look-ahead measured slower: 45-48 us against 43 for the
    // 4096 x 11008 forward at batch 8); two with MBT > 0, whose per-block
    // update lengthens the chain from load to use (measured 1-2 us faster
    // per 4096 x 11008 pass).  Loads use clamped in-range addresses; values
    // past the slice or past N are zeroed where they are multiplied.
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    constexpr int kAhead = UPD ? 2 : 1;
    constexpr int NA = UPD ? MBT : 1;
    float4v wq[kAhead][4], xq[kAhead], aq[kAhead][NA];
    // MBT > 0: G[b][n..n+3] of this lane's columns, fixed for the whole launch
    float4v gcol[NA];
#pragma unroll
    for (int b = 0; b < NA; ++b) gcol[b] = zero;
    if constexpr (UPD) {
#pragma unroll
        for (int b = 0; b < MBT; ++b)
            if (b < p.MB && nok) gcol[b] = ld4(p.grad + (int64_t)b * p.N + n);
    }
    auto fetch = [&](int k, float4v* wd, float4v& xd, float4v* ad) {
        const int kr = min(k + 4 * g, kw1 - 4);   // this lane group's 4 rows (K is a multiple of 4)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float* src = W + (int64_t)(kr + i) * p.N + (nok ? n : 0);
            if constexpr (UPD)
                wd[i] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(src));
            else
                wd[i] = ld4(src);
        }
        xd = ld4(X + kr);
        if constexpr (UPD) {
            // a[b][kr .. kr+3] of the previous step (rows past the batch are zero where used)
#pragma unroll
            for (int b = 0; b < MBT; ++b) ad[b] = ld4(p.act + (int64_t)min(b, p.MB - 1) * p.K + kr);
        }
    };
#pragma unroll
    for (int a = 0; a < kAhead; ++a)
        if (kw0 + 16 * a < kw1) fetch(kw0 + 16 * a, wq[a], xq[a], aq[a]);
    for (int k = kw0; k < kw1; k += 16 * kAhead) {
#pragma unroll
        for (int a = 0; a < kAhead; ++a) {
            const int kb = k + 16 * a;
            if (kb < kw1) {
                const bool ok = kb + 4 * g < kw1;
                float4v w[4], xv;
                if constexpr (UPD) {
                    // W' of rows kb+4g+i, columns n..n+3: the order of skinny_tn
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float4v d = zero;
#pragma unroll
                        for (int b = 0; b < MBT; ++b) {
                            const float av = b < p.MB ? aq[a][b][i] : 0.f;
#pragma unroll
                            for (int q = 0; q < 4; ++q) d[q] = fmaf(av, gcol[b][q], d[q]);
                        }
                        float4v u;
#pragma unroll
                        for (int q = 0; q < 4; ++q) u[q] = fmaf(-p.lr, d[q], wq[a][i][q]);
                        w[i] = (ok && nok) ? u : zero;
                    }
                    if (ok && nok) {
                        // non-temporal, as skinny_tn's: 16 lanes write a whole 256-byte
                        // segment of each row, and no later launch of the step re-reads W'
                        // soon enough for the last-level cache to hold it, where dirty
                        // lines would slow the next launches' reads
                        const int kr = kb + 4 * g;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            __builtin_nontemporal_store(w[i], reinterpret_cast<float4v*>(p.wout + (int64_t)(kr + i) * p.N + n));
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = (ok && nok) ? wq[a][i] : zero;
                }
                xv = (ok && mok) ? xq[a] : zero;
                if (kb + 16 * kAhead < kw1) fetch(kb + 16 * kAhead, wq[a], xq[a], aq[a]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i], w[i][q], acc[q], 0, 0, 0);
            }
        }
    }

    // acc[q][r] = out[m = 4g + r][n0 + 4j + q]; sum the waves in order 0..NW-1.
    if (wave > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave - 1][q][lane] = acc[q];
    }
    __syncthreads();
    if (wave != 0) {
        if (p.splits == 1) return;
    } else {
        for (int w = 0; w < NW - 1; ++w)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += red[w][q][lane];
    }

    if (p.splits > 1) {
        if (wave == 0 && nok) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g + r;
                if (m < p.MB) {
                    float* dst = p.partials + ((int64_t)split * p.MB + m) * p.N + n;
#pragma unroll
                    for (int q = 0; q < 4; ++q) store_coherent(dst + q, acc[q][r]);
                }
            }
        }
        if (!last_arrival(&p.tickets[cg], (unsigned)p.splits, &s_last)) return;
        if (wave != 0) return;
        // Add every split's partial, this workgroup's own included, in split
        // order.  Four splits' loads are issued at a time, unconditionally
        // (clamped in-range addresses; the extra ones are dropped), so that
        // none waits behind a branch.
        float4v sum[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] = {0.f, 0.f, 0.f, 0.f};
        const int nc = nok ? n : 0;
        for (int t0 = 0; t0 < p.splits; t0 += 4) {
            float x[4][4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = min(t0 + u, p.splits - 1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = min(4 * g + r, p.MB - 1);
                    const float* src = p.partials + ((int64_t)t * p.MB + m) * p.N + nc;
#pragma unroll
                    for (int q = 0; q < 4; ++q) x[u][r][q] = load_coherent(src + q);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int q = 0; q < 4; ++q) sum[q][r] += t0 + u < p.splits ? x[u][r][q] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = sum[q];
    }

    if (nok) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m >= p.MB) continue;
            const int64_t o = (int64_t)m * p.N + n;
            float4 v = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
            if constexpr (EPI == Epi::ReluMask) {
                uchar4 mk;
                mk.x = v.x > 0.f; mk.y = v.y > 0.f; mk.z = v.z > 0.f; mk.w = v.w > 0.f;
                v.x = relu_value(v.x); v.y = relu_value(v.y);
                v.z = relu_value(v.z); v.w = relu_value(v.w);
                *reinterpret_cast<uchar4*>(p.mask + o) = mk;
            }
            *reinterpret_cast<float4*>(p.C + o) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// dX and dW + SGD of one layer in a single pass over W (which both read):
//   out[b][k] = mask[b][k] * sum_n G[b][n] W[k][n]      (the old W)
//   W[k][n]  -= lr * sum_b a[b][k] G[b][n]              (or store the gradient)
// A workgroup of NW waves covers RG*16 rows of W; wave w takes the w-th slice
// of the columns, 32 at a time: lane group g takes columns n + 16h + 4g .. +3
// (h = 0, 1).  The dX MFMA has A = 16 rows of W and B = G^T (16 batch
// columns, zero past B): lane (i = lane%16, g) supplies W[k0 + i][c + q] and
// G[i][c + q] to MFMA q for its float4 at column c, so one float4 of each
// feeds four MFMAs; the waves' sums meet in LDS in wave order.  The update
// of those four elements comes from v_mfma_f32_16x16x4f32 as well: with
// A[m][j] = G[4s + j][n + 16h + m] and B[j][c] = a[4s + j][k0 + 16r + c], the
// 16x16 result D[m][c] = sum_j G a is dW^T of a 16 x 16 block, and lane
// (i, g) holds D[4g + e][i] = dW[k0 + 16r + i][n + 16h + 4g + e], exactly the
// float4 of W it loaded.  So each element of W is read once, feeds the dX
// reduction, and is written once, by the same lane.  Loads and stores of W
// are ordinary (cached): one instruction covers 64 bytes of each of 16 rows,
// and the L2 merges the two halves of every 128-byte line before it goes to
// HBM (non-temporal stores of half lines measured at half the bandwidth).
//
// When W has few rows (K / 16 row groups leave CUs idle), the columns are
// split too: workgroup (row group, column split cs) covers columns
// [cs * kchunk, (cs + 1) * kchunk); its dX sums are partial, go to
// partials [splits][B][K], and the last workgroup of the row group (integer
// ticket) adds them in split order before the mask.
template <int NW, int RG, int S, Epi EPI>
__global__ __launch_bounds__(NW * kWave) void skinny_ntu(SkinnyParams p) {
    __shared__ float4v red[NW - 1][RG][kWave];
    __shared__ int s_last;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rgroups = (p.K + 16 * RG - 1) / (16 * RG);
    const int rg = blockIdx.x % rgroups, cs = blockIdx.x / rgroups;
    const int k0 = rg * 16 * RG;
    const int i = lane & 15, g = lane >> 4;
    const bool bok = i < p.MB;
    if (p.loss && blockIdx.x == 0 && wave == 0) mean_rows_wave(p.rowloss, p.MB, p.inv_b, p.loss);
    const int cbeg = cs * p.kchunk, cend = min(p.N, cbeg + p.kchunk);
    const int nq = ((cend - cbeg + 32 * NW - 1) / (32 * NW)) * 32;   // slice, multiple of 32
    const int nbeg = cbeg + wave * nq;
    const int nend = min(cend, nbeg + nq);

    constexpr bool AD = EPI == Epi::Adapt;
    float4v acc[RG];
    const float* __restrict__ Wr[RG];
    float* __restrict__ Or[RG];
    float* __restrict__ Mr[RG];   // Adapt: moments of the same rows
    float* __restrict__ Vr[RG];
    bool rok[RG];
    float av[RG][S];   // a[4s + g][k0 + 16r + i]
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        acc[r] = {0.f, 0.f, 0.f, 0.f};
        const int krow = k0 + 16 * r + i;
        rok[r] = krow < p.K;
        Wr[r] = p.A + (int64_t)krow * p.N;
        Or[r] = p.wout + (int64_t)krow * p.N;
        Mr[r] = AD ? p.m + (int64_t)krow * p.N : nullptr;
        Vr[r] = AD ? p.v + (int64_t)krow * p.N : nullptr;
#pragma unroll
        for (int t = 0; t < S; ++t) {
            const int b = 4 * t + g;
            av[r][t] = (rok[r] && b < p.MB) ? p.act[(int64_t)b * p.K + krow] : 0.f;
        }
    }
    const float* __restrict__ Gr = p.B + (int64_t)(bok ? i : 0) * p.N;
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    // gv: G[i][cols] for the dX MFMA; gu: G[4s + g][n + 16h + i] for the update
    float4v gv[2], w[RG][2], gvn[2], wn[RG][2];
    float4v mo[RG][2], vo[RG][2], mon[RG][2], von[RG][2];   // Adapt: moments
    float gu[2][S], gun[2][S];
    auto fetch = [&](int n, float4v* gd, float4v (*wd)[2], float (*ud)[S], float4v (*md)[2], float4v (*vd)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = n + 16 * h + 4 * g;
            const bool cok = c < nend;   // N is a multiple of 4
            const float4v v = ld4(cok ? Gr + c : Gr);
            gd[h] = (cok && bok) ? v : zero;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const bool ok = cok && rok[r];
                const float4v x = ld4(ok ? Wr[r] + c : p.A);
                wd[r][h] = ok ? x : zero;
                if constexpr (AD) {
                    md[r][h] = ld4(ok ? Mr[r] + c : p.m);
                    vd[r][h] = ld4(ok ? Vr[r] + c : p.v);
                }
            }
            const int cu = n + 16 * h + i;
#pragma unroll
            for (int t = 0; t < S; ++t) {
                const int b = 4 * t + g;
                const bool ok = cu < nend && b < p.MB;
                const float x = p.B[ok ? (int64_t)b * p.N + cu : 0];
                ud[h][t] = ok ? x : 0.f;
            }
        }
    };
    if (nbeg < nend) fetch(nbeg, gvn, wn, gun, mon, von);
    for (int n = nbeg; n < nend; n += 32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            gv[h] = gvn[h];
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                w[r][h] = wn[r][h];
                if constexpr (AD) {
                    mo[r][h] = mon[r][h];
                    vo[r][h] = von[r][h];
                }
            }
#pragma unroll
            for (int t = 0; t < S; ++t) gu[h][t] = gun[h][t];
        }
        if (n + 32 < nend) fetch(n + 32, gvn, wn, gun, mon, von);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = n + 16 * h + 4 * g;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(w[r][h][q], gv[h][q], acc[r], 0, 0, 0);
                float4v d = zero;
#pragma unroll
                for (int t = 0; t < S; ++t) d = __builtin_amdgcn_mfma_f32_16x16x4f32(gu[h][t], av[r][t], d, 0, 0, 0);
                if (c < nend && rok[r]) {
                    float4v* dst = reinterpret_cast<float4v*>(Or[r] + c);
                    if constexpr (EPI == Epi::Sgd) {
                        *dst = w[r][h] - p.lr * d;
                    } else if constexpr (AD) {
                        float4v wv = w[r][h], mv = mo[r][h], vv = vo[r][h];
                        opt_apply4(p.opt, wv, d, mv, vv);
                        *dst = wv;
                        *reinterpret_cast<float4v*>(Mr[r] + c) = mv;
                        *reinterpret_cast<float4v*>(Vr[r] + c) = vv;
                    } else {
                        *dst = d;
                    }
                }
            }
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int r = 0; r < RG; ++r) red[wave - 1][r][lane] = acc[r];
    }
    __syncthreads();
    if (wave == 0) {
        for (int v = 0; v < NW - 1; ++v)
#pragma unroll
            for (int r = 0; r < RG; ++r) acc[r] += red[v][r][lane];
    }
    // acc[r][e] = out[b = lane%16][k = k0 + 16r + 4*(lane/16) + e]
    const int b = lane & 15;
    if (p.splits > 1) {
        if (wave == 0 && b < p.MB) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const int k = k0 + 16 * r + 4 * g;
                if (k >= p.K) continue;
                float* dst = p.partials + ((int64_t)cs * p.MB + b) * p.K + k;
#pragma unroll
                for (int e = 0; e < 4; ++e) store_coherent(dst + e, acc[r][e]);
            }
        }
        if (!last_arrival(&p.tickets[rg], (unsigned)p.splits, &s_last)) return;
        if (wave != 0 || b >= p.MB) return;
        // every split's partial, this workgroup's own included, in split
        // order; four splits' loads in flight at a time (clamped addresses,
        // the extra ones dropped)
#pragma unroll
        for (int r = 0; r < RG; ++r) {
            const int k = min(k0 + 16 * r + 4 * g, p.K - 4);
            float4v sum = {0.f, 0.f, 0.f, 0.f};
            for (int t0 = 0; t0 < p.splits; t0 += 4) {
                float x[4][4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float* src = p.partials + ((int64_t)min(t0 + u, p.splits - 1) * p.MB + b) * p.K + k;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[u][e] = load_coherent(src + e);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum[e] += t0 + u < p.splits ? x[u][e] : 0.f;
            }
            acc[r] = sum;
        }
    } else if (wave != 0) {
        return;
    }
    if (b >= p.MB) return;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const int k = k0 + 16 * r + 4 * g;
        if (k >= p.K) continue;
        const int64_t o = (int64_t)b * p.K + k;
        float4 v = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
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
// Each lane keeps G[0..B)[n..n+3] in registers and walks ROWS rows of W in
// chunks of 8 (the next chunk's loads are issued before the current chunk is
// updated); the per-row a[b][k] come from LDS.
template <int MB, int ROWS, Epi EPI>
__global__ __launch_bounds__(256) void skinny_tn(SkinnyParams p) {
    constexpr bool AD = EPI == Epi::Adapt;
    constexpr int CH = AD ? 4 : 8;   // Adapt streams W, m and v: fewer rows in flight
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
    float4v gv[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        gv[b] = {0.f, 0.f, 0.f, 0.f};
        if (b < p.MB) gv[b] = ld4(p.B + (int64_t)b * p.N + n);
    }
    const int rows = min(ROWS, p.K - k0);
    const int64_t off0 = (int64_t)k0 * p.N + n;
    float* base = p.C + off0;
    float* mbase = AD ? p.m + off0 : nullptr;
    float* vbase = AD ? p.v + off0 : nullptr;
    float4v w[2][CH], mo[2][CH], vo[2][CH];
    auto load_chunk = [&](int buf, int c0) {
#pragma unroll
        for (int r = 0; r < CH; ++r)
            if (c0 + r < rows) {
                const int64_t o = (int64_t)(c0 + r) * p.N;
                w[buf][r] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(base + o));
                if constexpr (AD) {
                    mo[buf][r] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(mbase + o));
                    vo[buf][r] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(vbase + o));
                }
            }
    };
    if constexpr (EPI == Epi::Sgd || AD) load_chunk(0, 0);
#pragma unroll
    for (int c0 = 0, buf = 0; c0 < ROWS; c0 += CH, buf ^= 1) {
        if (c0 >= rows) break;
        if constexpr (EPI == Epi::Sgd || AD) {
            if (c0 + CH < rows) load_chunk(buf ^ 1, c0 + CH);
        }
#pragma unroll
        for (int r = 0; r < CH; ++r) {
            const int rr = c0 + r;
            if (rr >= rows) break;
            // b ascending, one fma per b, then one fma for the step (the
            // fused pass in skinny_nn repeats exactly this arithmetic)
            float4v d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const float av = sa[rr][b];
#pragma unroll
                for (int q = 0; q < 4; ++q) d[q] = fmaf(av, gv[b][q], d[q]);
            }
            float* dst = base + (int64_t)rr * p.N;
            if constexpr (EPI == Epi::Sgd) {
                float4v v;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = fmaf(-p.lr, d[q], w[buf][r][q]);
                __builtin_nontemporal_store(v, reinterpret_cast<float4v*>(dst));
            } else if constexpr (AD) {
                float4v wv = w[buf][r], mv = mo[buf][r], vv = vo[buf][r];
                opt_apply4(p.opt, wv, d, mv, vv);
                const int64_t o = (int64_t)rr * p.N;
                __builtin_nontemporal_store(wv, reinterpret_cast<float4v*>(dst));
                __builtin_nontemporal_store(mv, reinterpret_cast<float4v*>(mbase + o));
                __builtin_nontemporal_store(vv, reinterpret_cast<float4v*>(vbase + o));
            } else {
                *reinterpret_cast<float4v*>(dst) = d;
            }
        }
    }
}

template <Epi EPI>
hipError_t go_ntu(const SkinnyLaunch& L, const SkinnyParams& p, hipStream_t s) {
    if (p.MB <= 4) hipLaunchKernelGGL((skinny_ntu<8, 1, 1, EPI>), dim3(L.grid), dim3(8 * 64), 0, s, p);
    else if (p.MB <= 8) hipLaunchKernelGGL((skinny_ntu<8, 1, 2, EPI>), dim3(L.grid), dim3(8 * 64), 0, s, p);
    else hipLaunchKernelGGL((skinny_ntu<8, 1, 4, EPI>), dim3(L.grid), dim3(8 * 64), 0, s, p);
    return hipGetLastError();
}

// rows of W per dW workgroup
constexpr int kTnRows = 32;

template <int MB>
hipError_t go_tn(const SkinnyLaunch& L, const SkinnyParams& p, hipStream_t s) {
    if (L.epi == Epi::Sgd)
        hipLaunchKernelGGL((skinny_tn<MB, kTnRows, Epi::Sgd>), dim3(L.grid), dim3(256), 0, s, p);
    else if (L.epi == Epi::Adapt)
        hipLaunchKernelGGL((skinny_tn<MB, kTnRows, Epi::Adapt>), dim3(L.grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((skinny_tn<MB, kTnRows, Epi::Grad>), dim3(L.grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int skinny_tn_rows() { return kTnRows; }

hipError_t launch_skinny(const SkinnyLaunch& L, const SkinnyParams& p, hipStream_t s) {
    if (p.MB < 1 || p.MB > 16) return hipErrorInvalidValue;
    switch (L.layout) {
    case Layout::NN:
        if (L.fused_update) {
            // previous step's dW + SGD of this W, then this forward (batch <= 8)
            if (L.waves != 8 || p.MB > 8 || !p.act || !p.grad || p.wout != p.B ||
                (L.epi != Epi::ReluMask && L.epi != Epi::Store))
                return hipErrorInvalidValue;
            if (p.MB <= 4) {
                if (L.epi == Epi::ReluMask)
                    hipLaunchKernelGGL((skinny_nn<8, Epi::ReluMask, 4>), dim3(L.grid), dim3(8 * 64), 0, s, p);
                else
                    hipLaunchKernelGGL((skinny_nn<8, Epi::Store, 4>), dim3(L.grid), dim3(8 * 64), 0, s, p);
            } else {
                if (L.epi == Epi::ReluMask)
                    hipLaunchKernelGGL((skinny_nn<8, Epi::ReluMask, 8>), dim3(L.grid), dim3(8 * 64), 0, s, p);
                else
                    hipLaunchKernelGGL((skinny_nn<8, Epi::Store, 8>), dim3(L.grid), dim3(8 * 64), 0, s, p);
            }
            return hipGetLastError();
        }
        if (L.waves == 8) {
            if (L.epi == Epi::ReluMask)
                hipLaunchKernelGGL((skinny_nn<8, Epi::ReluMask>), dim3(L.grid), dim3(8 * 64), 0, s, p);
            else
                hipLaunchKernelGGL((skinny_nn<8, Epi::Store>), dim3(L.grid), dim3(8 * 64), 0, s, p);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    case Layout::NT:
        if (L.fused_update) {
            // 16 rows of W per workgroup (measured at batch 8 over an
            // 11008 x 4096 W: 64.6 us against 76.8 with 32 rows and 67.5
            // with 64; 16-wave workgroups were slower)
            if (p.splits < 1 || p.kchunk < 1 || (int64_t)p.splits * p.kchunk < p.N ||
                (int64_t)(p.splits - 1) * p.kchunk >= p.N || L.grid != ((p.K + 15) / 16) * p.splits ||
                (p.splits > 1 && (!p.partials || !p.tickets)))
                return hipErrorInvalidValue;
            if (L.epi == Epi::Sgd) return go_ntu<Epi::Sgd>(L, p, s);
            if (L.epi == Epi::Adapt) return go_ntu<Epi::Adapt>(L, p, s);
            if (L.epi == Epi::Grad) return go_ntu<Epi::Grad>(L, p, s);
        }
        return hipErrorInvalidValue;
    case Layout::TN:
        if (p.MB <= 4) return go_tn<4>(L, p, s);
        if (p.MB <= 8) return go_tn<8>(L, p, s);
        return go_tn<16>(L, p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mlp
