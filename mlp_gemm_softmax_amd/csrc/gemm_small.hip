// Float32 MFMA GEMM for small, under-filled products (a few hundred output
// tiles at most, e.g. the batch-32/1024 MLP's 1024x128x784 forward and
// 784x128x1024 dW).  Splitting K across workgroups costs two extra memory
// round trips (partials out with device-scope stores, back in by the last
// workgroup), which dominates such products; here the K split stays inside a
// workgroup instead:
//   - a workgroup of NW waves owns one 32x32 output tile;
//   - wave w accumulates the w-th slice of K with v_mfma_f32_32x32x2f32,
//     loading its MFMA operands straight from global memory (L2) into
//     registers, several 8-k chunks ahead of the MFMAs -- no LDS staging and
//     no barriers in the K loop;
//   - the NW accumulators meet in LDS and are added in wave order 0..NW-1,
//     then the fused epilogue is applied.
// Operand k map (same for A and B, which is all the reduction needs): in
// chunk c, lanes 0-31 hold k = 8c..8c+3 and lanes 32-63 hold k = 8c+4..8c+7,
// and MFMA q (0..3) takes the q-th of those four values.
#include "kernels.hpp"
#include "epilogue1.hpp"
#include "head_body.hpp"
#include "tail.hpp"

namespace mlp {
namespace {

constexpr int kDepth = 8;   // chunks of 8 k in flight per wave

// The four k-values of chunk c (k = k0 + 4h + 0..3) for row r of an operand.
// KC: element (r, k) at g + r*ld + k (16-byte load when VEC == 4);
// otherwise at g + k*ld + r (four 4-byte loads, coalesced across lanes).
// Rows and k past the matrix are read from clamped in-range addresses and
// the values are used as they are: rows past M or N only reach outputs that
// are never stored, and the k tail is zeroed where the chunk is multiplied.
// Keeping the loads free of selects and branches lets the loads of all
// chunks stay in flight together.
template <bool KC, int VEC>
__device__ __forceinline__ float4v load_op(const float* __restrict__ g, int64_t ld, int r, int rmax,
                                           int k, int kmax) {
    const int64_t rc = r < rmax ? r : rmax - 1;
    if constexpr (KC && VEC == 4) {
        return *reinterpret_cast<const float4v*>(g + rc * ld + (k < kmax ? k : 0));   // kmax % 4 == 0
    } else {
        float4v v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t kc = k + q < kmax ? k + q : kmax - 1;
            v[q] = KC ? g[rc * ld + kc] : g[kc * ld + rc];
        }
        return v;
    }
}


template <int NW, Layout LAY, int VEC, Epi EPI>
__global__ __launch_bounds__(NW * 64) void gemm_small_kernel(GemmParams p) {
    constexpr bool AKC = LAY != Layout::TN;   // A stored [M][K]
    constexpr bool BKC = LAY == Layout::NT;   // B stored [N][K]
    __shared__ float red[NW][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_n = (p.N + 31) / 32;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (id / tiles_n) * 32, n0 = (id % tiles_n) * 32;
    const int h = lane >> 5;
    const int ra = m0 + (lane & 31), rb = n0 + (lane & 31);

    // this wave's K slice, in whole chunks of 8
    const int chunks = (p.K + 7) / 8;
    const int per = (chunks + NW - 1) / NW;
    const int c0 = wave * per, c1 = min(chunks, c0 + per);

    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    float16v acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;

    float4v qa[kDepth], qb[kDepth];
    if (c0 < c1) {
        // chunks past this wave's slice load a clamped chunk and are never used
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int k = 8 * min(c0 + d, c1 - 1) + 4 * h;
            qa[d] = load_op<AKC, VEC>(A, p.lda, ra, p.M, k, p.K);
            qb[d] = load_op<BKC, VEC>(B, p.ldb, rb, p.N, k, p.K);
        }
    }
    for (int c = c0; c < c1; c += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (c + d < c1) {
                float4v a = qa[d], b = qb[d];
                if (8 * (c + d) + 8 > p.K) {   // the chunk holding the k tail
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bool kok = 8 * (c + d) + 4 * h + q < p.K;
                        a[q] = kok ? a[q] : 0.f;
                        b[q] = kok ? b[q] : 0.f;
                    }
                }
                const int cn = c + d + kDepth;
                if (cn < c1) {
                    const int k = 8 * cn + 4 * h;
                    qa[d] = load_op<AKC, VEC>(A, p.lda, ra, p.M, k, p.K);
                    qb[d] = load_op<BKC, VEC>(B, p.ldb, rb, p.N, k, p.K);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    // 1024 outputs of the tile; thread t takes lane position t%64 and
    // registers r = t/64, t/64 + NW, ... (acc element r of lane l sits at
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32).
    for (int e = threadIdx.x; e < 16 * 64; e += NW * 64) {
        const int r = e / 64, l = e % 64;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += red[w][r][l];
        const int row = m0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int col = n0 + (l & 31);
        if (row < p.M && col < p.N) epilogue<EPI>(p, row, col, v);
    }
}

// The same scheme with 32 x 16 tiles on v_mfma_f32_16x16x4f32, twice as many
// workgroups for the same product (the f32 matrix-core time of one CU, not
// latency, bounds a 32 x 32 tile of a K = 784 product).  A chunk is 16 k:
// lane (i = lane%16, g = lane/16) loads k = k0 + 4g .. +3 of A rows
// m0 + i and m0 + 16 + i and of B column n0 + i, and MFMA q (0..3) takes
// component q of each, so one 16-byte (or four coalesced 4-byte) load feeds
// four MFMAs.  Result lane l holds rows 4(l/16)..+3 of column l%16.
template <bool KC, int VEC>
__device__ __forceinline__ float4v load_op16(const float* __restrict__ g, int64_t ld, int r, int rmax, int k,
                                             int kmax) {
    const int64_t rc = r < rmax ? r : rmax - 1;
    if constexpr (KC && VEC == 4) {
        return *reinterpret_cast<const float4v*>(g + rc * ld + (k < kmax ? k : 0));   // kmax % 4 == 0
    } else {
        float4v v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t kc = k + q < kmax ? k + q : kmax - 1;
            v[q] = KC ? g[rc * ld + kc] : g[kc * ld + rc];
        }
        return v;
    }
}

// With TAIL, the first tail_jobs(t.H) workgroups run the fused output
// layer's tail jobs (tail.hpp) instead of tiles.  With HEAD (forward of the
// last hidden layer, ReluMask, 16 waves), the activations and masks go out
// with device-scope stores, and the workgroup that finishes the last column
// tile of a 32-row block (integer ticket per row block) runs the output
// layer's head for those rows (head_body.hpp) with dynamic LDS.
template <int NW, Layout LAY, int VEC, Epi EPI, bool TAIL, bool HEAD>
__global__ __launch_bounds__(NW * 64) void gemm_small16_kernel(GemmParams p, TailParams t, HeadParams hp) {
    constexpr bool AKC = LAY != Layout::TN;   // A stored [M][K]
    constexpr bool BKC = LAY == Layout::NT;   // B stored [N][K]
    constexpr int D = kDepth / 2;             // chunks of 16 k in flight per wave
    static_assert(!HEAD || (NW == kHeadWaves && EPI == Epi::ReluMask && LAY == Layout::NN), "head layout");
    __shared__ float4v red[NW][2][64];
    __shared__ int s_last;
    extern __shared__ float head_lds[];
    int bid = blockIdx.x, nb = gridDim.x;
    if constexpr (TAIL) {
        const int jobs = tail_jobs(t.H);
        if (bid < jobs) {
            tail_job<NW>(t, bid, &red[0][0][0]);
            return;
        }
        bid -= jobs;
        nb -= jobs;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tiles_n = (p.N + 15) / 16;
    const int id = xcd_remap(bid, nb);
    const int m0 = (id / tiles_n) * 32, n0 = (id % tiles_n) * 16;
    const int i = lane & 15, g = lane >> 4;

    const int chunks = (p.K + 15) / 16;
    const int per = (chunks + NW - 1) / NW;
    const int c0 = wave * per, c1 = min(chunks, c0 + per);

    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    float4v acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float4v qa[D][2], qb[D];
    auto fetch = [&](int d, int c) {
        const int k = 16 * c + 4 * g;
        qa[d][0] = load_op16<AKC, VEC>(A, p.lda, m0 + i, p.M, k, p.K);
        qa[d][1] = load_op16<AKC, VEC>(A, p.lda, m0 + 16 + i, p.M, k, p.K);
        qb[d] = load_op16<BKC, VEC>(B, p.ldb, n0 + i, p.N, k, p.K);
    };
    if (c0 < c1) {
        // chunks past this wave's slice load a clamped chunk and are never used
#pragma unroll
        for (int d = 0; d < D; ++d) fetch(d, min(c0 + d, c1 - 1));
    }
    for (int c = c0; c < c1; c += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (c + d < c1) {
                float4v a0 = qa[d][0], a1 = qa[d][1], b = qb[d];
                if (16 * (c + d) + 16 > p.K) {   // the chunk holding the k tail
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bool kok = 16 * (c + d) + 4 * g + q < p.K;
                        a0[q] = kok ? a0[q] : 0.f;
                        a1[q] = kok ? a1[q] : 0.f;
                        b[q] = kok ? b[q] : 0.f;
                    }
                }
                if (c + d + D < c1) fetch(d, c + d + D);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[q], b[q], acc[0], 0, 0, 0);
                    acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[q], b[q], acc[1], 0, 0, 0);
                }
            }
        }
    }

    red[wave][0][lane] = acc[0];
    red[wave][1][lane] = acc[1];
    __syncthreads();
    // 512 outputs: thread t < 128 takes row block t/64 and lane position t%64
    // and adds the waves' float4s in wave order 0..NW-1.
    if (threadIdx.x < 128) {
        const int rbk = threadIdx.x >> 6, l = threadIdx.x & 63;
        float4v v = red[0][rbk][l];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += red[w][rbk][l];
        const int col = n0 + (l & 15);
        if constexpr (EPI == Epi::Softmax) {
            // One column tile holds every class (N <= 16): the 16 lanes of a
            // DPP row hold the same four rows, columns 0..15, so each row's
            // max and sum are 16-lane reductions (columns past N masked).
            const bool cok = col < p.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + 16 * rbk + 4 * (l >> 4) + e;
                const float z = cok ? v[e] : -INFINITY;
                const float mx = row16_max(z);
                const float ex = cok ? expf(z - mx) : 0.f;
                const float se = row16_sum(ex);
                if (row < p.M && cok) p.C[(int64_t)row * p.ldc + col] = ex / se;
            }
        } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = m0 + 16 * rbk + 4 * (l >> 4) + e;
            if (row < p.M && col < p.N) {
                if constexpr (HEAD) {
                    const int64_t o = (int64_t)row * p.ldc + col;
                    const bool pos = v[e] > 0.f;
                    store_coherent(p.C + o, relu_value(v[e]));
                    store_coherent(p.mask + o, (uint8_t)(pos ? 1 : 0));
                } else {
                    epilogue<EPI>(p, row, col, v[e]);
                }
            }
        }
        }
    }
    if constexpr (HEAD) {
        if (!last_arrival(&p.tickets[m0 / 32], (unsigned)tiles_n, &s_last)) return;
        head_block<true>(hp, m0, head_lds, reinterpret_cast<float4v(*)[kWave]>(&red[0][0][0]));
    }
}

template <int NW, Layout LAY, int VEC, Epi EPI>
hipError_t go(const GemmParams& p, int grid, bool t16, hipStream_t st) {
    const TailParams none{};
    const HeadParams nohead{};
    if (t16)
        hipLaunchKernelGGL((gemm_small16_kernel<NW, LAY, VEC, EPI, false, false>), dim3(grid), dim3(NW * 64), 0, st,
                           p, none, nohead);
    else
        hipLaunchKernelGGL((gemm_small_kernel<NW, LAY, VEC, EPI>), dim3(grid), dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

template <int NW, int VEC, Epi EPI>
hipError_t go_tail(const GemmParams& p, int grid, const TailParams& t, hipStream_t st) {
    const HeadParams nohead{};
    hipLaunchKernelGGL((gemm_small16_kernel<NW, Layout::TN, VEC, EPI, true, false>), dim3(grid + tail_jobs(t.H)),
                       dim3(NW * 64), 0, st, p, t, nohead);
    return hipGetLastError();
}

template <int NW>
hipError_t dispatch_tail(const GemmLaunch& L, const GemmParams& p, const TailParams& t, hipStream_t st) {
    if (L.epi == Epi::Sgd)
        return L.vec == 4 ? go_tail<NW, 4, Epi::Sgd>(p, L.grid, t, st) : go_tail<NW, 1, Epi::Sgd>(p, L.grid, t, st);
    if (L.epi == Epi::Adapt)
        return L.vec == 4 ? go_tail<NW, 4, Epi::Adapt>(p, L.grid, t, st) : go_tail<NW, 1, Epi::Adapt>(p, L.grid, t, st);
    if (L.epi == Epi::Grad)
        return L.vec == 4 ? go_tail<NW, 4, Epi::Grad>(p, L.grid, t, st) : go_tail<NW, 1, Epi::Grad>(p, L.grid, t, st);
    return hipErrorInvalidValue;
}

template <int NW, Layout LAY, Epi EPI>
hipError_t go_vec(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    const bool t16 = L.cfg == TileCfg::T32x16;
    return L.vec == 4 ? go<NW, LAY, 4, EPI>(p, L.grid, t16, st) : go<NW, LAY, 1, EPI>(p, L.grid, t16, st);
}

template <int NW>
hipError_t go_softmax(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    const TailParams none{};
    const HeadParams nohead{};
    if (L.vec == 4)
        hipLaunchKernelGGL((gemm_small16_kernel<NW, Layout::NN, 4, Epi::Softmax, false, false>), dim3(L.grid),
                           dim3(NW * 64), 0, st, p, none, nohead);
    else
        hipLaunchKernelGGL((gemm_small16_kernel<NW, Layout::NN, 1, Epi::Softmax, false, false>), dim3(L.grid),
                           dim3(NW * 64), 0, st, p, none, nohead);
    return hipGetLastError();
}

template <int NW>
hipError_t dispatch(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    switch (L.layout) {
    case Layout::NN:
        if (L.epi == Epi::ReluMask) return go_vec<NW, Layout::NN, Epi::ReluMask>(L, p, st);
        if (L.epi == Epi::Store) return go_vec<NW, Layout::NN, Epi::Store>(L, p, st);
        break;
    case Layout::NT:
        if (L.epi == Epi::MaskMul) return go_vec<NW, Layout::NT, Epi::MaskMul>(L, p, st);
        break;
    case Layout::TN:
        if (L.epi == Epi::Sgd) return go_vec<NW, Layout::TN, Epi::Sgd>(L, p, st);
        if (L.epi == Epi::Adapt) return go_vec<NW, Layout::TN, Epi::Adapt>(L, p, st);
        if (L.epi == Epi::Grad) return go_vec<NW, Layout::TN, Epi::Grad>(L, p, st);
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

// Waves per workgroup for a small product: the fewest (4, 8 or 16) whose K
// slices fit one prefetch window (every load of a wave in flight at once),
// else 16.
int gemm_small_waves(int M, int N, int K) {
    (void)M;
    (void)N;
    const int chunks = (K + 7) / 8;
    for (int nw : {4, 8, 16})
        if ((chunks + nw - 1) / nw <= kDepth) return nw;
    return 16;
}

hipError_t launch_gemm_small_head(const GemmLaunch& L, const GemmParams& p, const HeadParams& hp,
                                  hipStream_t st) {
    if (L.bf16 || p.Cb || L.cfg != TileCfg::T32x16 || L.layout != Layout::NN || L.epi != Epi::ReluMask ||
        hp.RB != 32 || !p.tickets)
        return hipErrorInvalidValue;
    const TailParams none{};
    const size_t lds = head_lds_bytes(hp.H, hp.C, hp.RB);
    if (L.vec == 4)
        hipLaunchKernelGGL((gemm_small16_kernel<kHeadWaves, Layout::NN, 4, Epi::ReluMask, false, true>),
                           dim3(L.grid), dim3(kHeadThreads), lds, st, p, none, hp);
    else
        hipLaunchKernelGGL((gemm_small16_kernel<kHeadWaves, Layout::NN, 1, Epi::ReluMask, false, true>),
                           dim3(L.grid), dim3(kHeadThreads), lds, st, p, none, hp);
    return hipGetLastError();
}

hipError_t launch_gemm_small_tail(const GemmLaunch& L, const GemmParams& p, int waves, const TailParams& t,
                                  hipStream_t st) {
    if (L.bf16 || p.Cb || L.cfg != TileCfg::T32x16 || L.layout != Layout::TN) return hipErrorInvalidValue;
    switch (waves) {
    case 4: return dispatch_tail<4>(L, p, t, st);
    case 8: return dispatch_tail<8>(L, p, t, st);
    case 16: return dispatch_tail<16>(L, p, t, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_small(const GemmLaunch& L, const GemmParams& p, int waves, hipStream_t st) {
    if (L.bf16 || p.Cb) return hipErrorInvalidValue;
    if (L.epi == Epi::Softmax) {
        // probabilities straight from the logits product: one 16-column tile
        if (L.cfg != TileCfg::T32x16 || L.layout != Layout::NN || p.N > 16 || p.N < 1 ||
            L.grid != (p.M + 31) / 32)
            return hipErrorInvalidValue;
        switch (waves) {
        case 4: return go_softmax<4>(L, p, st);
        case 8: return go_softmax<8>(L, p, st);
        case 16: return go_softmax<16>(L, p, st);
        }
        return hipErrorInvalidValue;
    }
    switch (waves) {
    case 4: return dispatch<4>(L, p, st);
    case 8: return dispatch<8>(L, p, st);
    case 16: return dispatch<16>(L, p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace mlp
