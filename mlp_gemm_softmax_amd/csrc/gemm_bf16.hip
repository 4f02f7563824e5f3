// bf16-operand MFMA GEMM (float32 accumulate) for the fast-path contract:
// v_mfma_f32_32x32x16_bf16, 1024 flop/clk per SIMD on gfx950.  Same three
// layouts, epilogues and deterministic split-K as the float32 kernel; the
// epilogues still see the float32 accumulator (the ReLU mask is taken from
// it), and outputs are rounded to bf16 only where a later GEMM consumes them.
//
// LDS tiles are k-contiguous bf16 [row][k] with a 72-element (144-byte) row
// stride; each MFMA operand is one 16-byte read per lane: lanes 0-31 take
// k = 16c..16c+7 and lanes 32-63 take k = 16c+8..16c+15 of row lane%32.
#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;     // bf16 elements per LDS row

template <int BM_, int BN_, int WM_, int WN_>
struct Shape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
};

// k-contiguous operand; VEC = 8 loads 16 bytes (8 bf16) per access.
template <int R, int VEC>
struct KLoad {
    static constexpr int PER = R * kBK / (kThreads * VEC);
    static_assert(PER >= 1, "tile too small for the loader");
    uint32_t v[VEC == 8 ? PER * 4 : PER];

    __device__ __forceinline__ void load(const bf16_t* __restrict__ g, int64_t ld, int r0,
                                         int rmax, int k0, int kmax, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + kThreads * i;
            if constexpr (VEC == 8) {
                const int row = idx / (kBK / 8), kq = idx % (kBK / 8);
                const int r = r0 + row, k = k0 + 8 * kq;
                uint4 x = make_uint4(0u, 0u, 0u, 0u);
                if (r < rmax && k < kmax) x = *reinterpret_cast<const uint4*>(g + (int64_t)r * ld + k);
                v[4 * i + 0] = x.x;
                v[4 * i + 1] = x.y;
                v[4 * i + 2] = x.z;
                v[4 * i + 3] = x.w;
            } else {
                const int row = idx / kBK, kk = idx % kBK;
                const int r = r0 + row, k = k0 + kk;
                v[i] = (r < rmax && k < kmax) ? (uint32_t)g[(int64_t)r * ld + k] : 0u;
            }
        }
    }
    __device__ __forceinline__ void store(bf16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int idx = tid + kThreads * i;
            if constexpr (VEC == 8) {
                const int row = idx / (kBK / 8), kq = idx % (kBK / 8);
                *reinterpret_cast<uint4*>(s + row * kLDK + 8 * kq) =
                    make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
            } else {
                const int row = idx / kBK, kk = idx % kBK;
                s[row * kLDK + kk] = (bf16_t)v[i];
            }
        }
    }
};

// r-contiguous operand (element (r,k) at g + k*ld + r): lanes along r, each
// gathers KPT consecutive k into packed pairs and writes 16-byte runs along k.
template <int R>
struct MNLoad {
    static constexpr int KG = kThreads / R;
    static constexpr int KPT = kBK / KG;
    static_assert(KPT % 8 == 0, "k per thread must fill 16-byte runs");
    uint32_t v[KPT / 2];

    __device__ __forceinline__ void load(const bf16_t* __restrict__ g, int64_t ld, int r0,
                                         int rmax, int k0, int kmax, int tid) {
        const int r = r0 + tid % R, grp = tid / R;
        const bool rok = r < rmax;
#pragma unroll
        for (int i = 0; i < KPT / 2; ++i) {
            const int k = k0 + grp * KPT + 2 * i;
            const uint32_t lo = (rok && k < kmax) ? (uint32_t)g[(int64_t)k * ld + r] : 0u;
            const uint32_t hi = (rok && k + 1 < kmax) ? (uint32_t)g[(int64_t)(k + 1) * ld + r] : 0u;
            v[i] = lo | (hi << 16);
        }
    }
    __device__ __forceinline__ void store(bf16_t* s, int tid) const {
        const int r = tid % R, grp = tid / R;
#pragma unroll
        for (int q = 0; q < KPT / 8; ++q)
            *reinterpret_cast<uint4*>(s + r * kLDK + grp * KPT + 8 * q) =
                make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
};

template <Epi EPI>
__device__ __forceinline__ void epilogue(const GemmParams& p, int row, int col, float v) {
    const int64_t o = (int64_t)row * p.ldc + col;
    if constexpr (EPI == Epi::Store || EPI == Epi::Grad) {
        p.C[o] = v;
    } else if constexpr (EPI == Epi::ReluMask) {
        const bool pos = v > 0.f;
        const float a = pos ? v : 0.f;
        if (p.Cb) p.Cb[o] = f32_to_bf16(a); else p.C[o] = a;
        p.mask[o] = pos ? 1 : 0;
    } else if constexpr (EPI == Epi::MaskMul) {
        const float g = p.mask[o] ? v : 0.f;
        if (p.Cb) p.Cb[o] = f32_to_bf16(g); else p.C[o] = g;
    } else if constexpr (EPI == Epi::Sgd) {
        const float w = p.C[o] - p.lr * v;
        p.C[o] = w;
        if (p.Cb) p.Cb[o] = f32_to_bf16(w);
    }
}

template <class S, Layout LAY, int VEC, Epi EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_kernel(GemmParams p) {
    constexpr int BM = S::BM, BN = S::BN, FM = S::FM, FN = S::FN;
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][BM * kLDK];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][BN * kLDK];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

    const int ntile = p.tiles_m * p.tiles_n;
    const int id = xcd_remap(blockIdx.x, gridDim.x);
    const int split = id / ntile;
    const int tile = id % ntile;
    int tm, tn;
    {
        constexpr int GROUP = 8;
        const int width = GROUP * p.tiles_n;
        const int first = (tile / width) * GROUP;
        const int gs = min(p.tiles_m - first, GROUP);
        const int in = tile % width;
        tm = first + in % gs;
        tn = in / gs;
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

    const bf16_t* A = static_cast<const bf16_t*>(p.A);
    const bf16_t* B = static_cast<const bf16_t*>(p.B);

    using ALoad = typename std::conditional<LAY == Layout::TN, MNLoad<BM>, KLoad<BM, VEC>>::type;
    using BLoad = typename std::conditional<LAY == Layout::NT, KLoad<BN, VEC>, MNLoad<BN>>::type;
    ALoad la;
    BLoad lb;

    float16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
        la.load(A, p.lda, m0, p.M, kbeg, kend, tid);
        lb.load(B, p.ldb, n0, p.N, kbeg, kend, tid);
        la.store(sA[0], tid);
        lb.store(sB[0], tid);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                la.load(A, p.lda, m0, p.M, kbeg + (kt + 1) * kBK, kend, tid);
                lb.load(B, p.ldb, n0, p.N, kbeg + (kt + 1) * kBK, kend, tid);
            }
            const bf16_t* a_base = sA[cur] + (wm * S::WM + (lane & 31)) * kLDK + 8 * (lane >> 5);
            const bf16_t* b_base = sB[cur] + (wn * S::WN + (lane & 31)) * kLDK + 8 * (lane >> 5);
#pragma unroll
            for (int c = 0; c < kBK / 16; ++c) {
                bf16x8v a[FM], b[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a[i] = *reinterpret_cast<const bf16x8v*>(a_base + i * 32 * kLDK + 16 * c);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    b[j] = *reinterpret_cast<const bf16x8v*>(b_base + j * 32 * kLDK + 16 * c);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
            if (more) {
                la.store(sA[cur ^ 1], tid);
                lb.store(sB[cur ^ 1], tid);
            }
            __syncthreads();
        }
    }

    const int row_w = m0 + wm * S::WM + 4 * (lane >> 5);
    const int col_w = n0 + wn * S::WN + (lane & 31);

    if (p.splits > 1) {
        // Deterministic split-K (see the float32 kernel).
        float* part = p.partials + (int64_t)split * p.M * p.N;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row_w + i * 32 + 8 * (r >> 2) + (r & 3);
                    const int col = col_w + j * 32;
                    if (row < p.M && col < p.N) store_coherent(part + (int64_t)row * p.N + col, acc[i][j][r]);
                }
        if (!last_arrival(&p.tickets[tile], (unsigned)p.splits, &s_last)) return;
        float16v sum[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sum[i][j][r] = 0.f;
        for (int t = 0; t < p.splits; ++t) {
            const float* q = p.partials + (int64_t)t * p.M * p.N;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = row_w + i * 32 + 8 * (r >> 2) + (r & 3);
                        const int col = col_w + j * 32;
                        float v = acc[i][j][r];
                        if (t != split && row < p.M && col < p.N)
                            v = load_coherent(q + (int64_t)row * p.N + col);
                        sum[i][j][r] += v;
                    }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = sum[i][j];
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row_w + i * 32 + 8 * (r >> 2) + (r & 3);
                const int col = col_w + j * 32;
                if (row < p.M && col < p.N) epilogue<EPI>(p, row, col, acc[i][j][r]);
            }
}

template <class S, Layout LAY, int VEC, Epi EPI>
hipError_t go(const GemmParams& p, int grid, hipStream_t st) {
    hipLaunchKernelGGL((gemm_bf16_kernel<S, LAY, VEC, EPI>), dim3(grid), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <class S>
hipError_t dispatch_shape(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    const bool v8 = L.vec == 8;
    switch (L.layout) {
    case Layout::NN:
        if (L.epi == Epi::ReluMask)
            return v8 ? go<S, Layout::NN, 8, Epi::ReluMask>(p, L.grid, st)
                      : go<S, Layout::NN, 1, Epi::ReluMask>(p, L.grid, st);
        if (L.epi == Epi::Store)
            return v8 ? go<S, Layout::NN, 8, Epi::Store>(p, L.grid, st)
                      : go<S, Layout::NN, 1, Epi::Store>(p, L.grid, st);
        break;
    case Layout::NT:
        if (L.epi == Epi::MaskMul)
            return v8 ? go<S, Layout::NT, 8, Epi::MaskMul>(p, L.grid, st)
                      : go<S, Layout::NT, 1, Epi::MaskMul>(p, L.grid, st);
        if (L.epi == Epi::Store)
            return v8 ? go<S, Layout::NT, 8, Epi::Store>(p, L.grid, st)
                      : go<S, Layout::NT, 1, Epi::Store>(p, L.grid, st);
        break;
    case Layout::TN:
        if (L.epi == Epi::Sgd) return go<S, Layout::TN, 1, Epi::Sgd>(p, L.grid, st);
        if (L.epi == Epi::Grad) return go<S, Layout::TN, 1, Epi::Grad>(p, L.grid, st);
        break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    switch (L.cfg) {
    case TileCfg::T128x128: return dispatch_shape<Shape<128, 128, 64, 64>>(L, p, st);
    case TileCfg::T64x64: return dispatch_shape<Shape<64, 64, 32, 32>>(L, p, st);
    case TileCfg::T32x128: return dispatch_shape<Shape<32, 128, 32, 32>>(L, p, st);
    case TileCfg::T128x32: return dispatch_shape<Shape<128, 32, 32, 32>>(L, p, st);
    case TileCfg::T128x64: return dispatch_shape<Shape<128, 64, 64, 32>>(L, p, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace mlp
