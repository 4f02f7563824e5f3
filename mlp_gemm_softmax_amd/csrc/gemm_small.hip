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

namespace mlp {
namespace {

constexpr int kDepth = 8;   // chunks of 8 k in flight per wave

// The four k-values of chunk c (k = k0 + 4h + 0..3) for row r of an operand.
// KC: element (r, k) at g + r*ld + k (16-byte load when VEC == 4);
// otherwise at g + k*ld + r (four 4-byte loads, coalesced across lanes).
template <bool KC, int VEC>
__device__ __forceinline__ float4v load_op(const float* __restrict__ g, int64_t ld, int r, int rmax,
                                           int k, int kmax) {
    float4v v = {0.f, 0.f, 0.f, 0.f};
    if (r >= rmax) return v;
    if constexpr (KC && VEC == 4) {
        if (k < kmax) v = *reinterpret_cast<const float4v*>(g + (int64_t)r * ld + k);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (k + q < kmax) v[q] = KC ? g[(int64_t)r * ld + k + q] : g[(int64_t)(k + q) * ld + r];
    }
    return v;
}

template <Epi EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, int row, int col, float v) {
    const int64_t o = (int64_t)row * p.ldc + col;
    if constexpr (EPI == Epi::Store || EPI == Epi::Grad) {
        p.C[o] = v;
    } else if constexpr (EPI == Epi::ReluMask) {
        const bool pos = v > 0.f;
        p.C[o] = pos ? v : 0.f;
        p.mask[o] = pos ? 1 : 0;
    } else if constexpr (EPI == Epi::MaskMul) {
        p.C[o] = p.mask[o] ? v : 0.f;
    } else if constexpr (EPI == Epi::Sgd) {
        p.C[o] = p.C[o] - p.lr * v;
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
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
        const int k = 8 * (c0 + d) + 4 * h;
        if (c0 + d < c1) {
            qa[d] = load_op<AKC, VEC>(A, p.lda, ra, p.M, k, p.K);
            qb[d] = load_op<BKC, VEC>(B, p.ldb, rb, p.N, k, p.K);
        }
    }
    for (int c = c0; c < c1; c += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (c + d < c1) {
                const float4v a = qa[d], b = qb[d];
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

template <int NW, Layout LAY, int VEC, Epi EPI>
hipError_t go(const GemmParams& p, int grid, hipStream_t st) {
    hipLaunchKernelGGL((gemm_small_kernel<NW, LAY, VEC, EPI>), dim3(grid), dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

template <int NW, Layout LAY, Epi EPI>
hipError_t go_vec(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    return L.vec == 4 ? go<NW, LAY, 4, EPI>(p, L.grid, st) : go<NW, LAY, 1, EPI>(p, L.grid, st);
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

hipError_t launch_gemm_small(const GemmLaunch& L, const GemmParams& p, int waves, hipStream_t st) {
    if (L.bf16 || p.Cb) return hipErrorInvalidValue;
    switch (waves) {
    case 4: return dispatch<4>(L, p, st);
    case 8: return dispatch<8>(L, p, st);
    case 16: return dispatch<16>(L, p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace mlp
