// bf16-operand MFMA GEMM (float32 accumulate) for the fast-path contract:
// v_mfma_f32_32x32x16_bf16, 1024 flop/clk per SIMD on gfx950.  Same three
// layouts, epilogues and deterministic split-K as the float32 kernel; the
// epilogues still see the float32 accumulator (the ReLU mask is taken from
// it), and outputs are rounded to bf16 only where a later GEMM consumes them.
//
// Operand tiles keep their global orientation in LDS (16-byte copies):
//   k-contiguous operand: LDS [r][k], row stride 72 bf16; an MFMA operand is
//     one 16-byte read: lanes 0-31 take k = 16c..16c+7 and lanes 32-63 take
//     k = 16c+8..16c+15 of row lane%32;
//   r-contiguous operand: LDS [k][r], row stride R+16 bf16; the same eight
//     k-values per lane come from two ds_read_b64_tr_b16 transpose reads.
//     Within each 16-lane group that instruction hands lane i element i%4 of
//     the 8-byte chunks addressed by lanes 4e+i/4 (e = 0..3); pointing lane s
//     at row kb + s/4, columns m0 + 4(s%4) therefore gives lane i the four
//     values k = kb..kb+3 of row m0 + i.
#include "kernels.hpp"
#include "epilogue1.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

template <int BM_, int BN_, int WM_, int WN_>
struct Shape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
};

// Operand tile of R rows x kBK k in bf16.  KC: stored k-contiguous (element
// (r,k) at g + r*ld + k), else r-contiguous (at g + k*ld + r).  VEC: 8 =
// 16-byte global loads (contiguous extent and ld multiples of 8), 1 = 2-byte.
template <int R, bool KC, int VEC>
struct Tile {
    static constexpr int LD = KC ? kBK + 8 : R + 16;         // LDS row stride (bf16)
    static constexpr int ELEMS = KC ? R * LD : kBK * LD;     // LDS bf16 per stage
    static constexpr int CONT = KC ? kBK : R;
    static constexpr int PER = R * kBK / (kThreads * VEC);
    static_assert(PER >= 1, "tile too small for the loader");
    uint32_t v[VEC == 8 ? PER * 4 : PER];

    __device__ __forceinline__ static void where(int tid, int i, int& line, int& off) {
        const int idx = tid + kThreads * i;
        line = idx / (CONT / VEC);
        off = (idx % (CONT / VEC)) * VEC;
    }

    __device__ __forceinline__ void load(const bf16_t* __restrict__ g, int64_t ld, int r0, int rmax,
                                         int k0, int kmax, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int line, off;
            where(tid, i, line, off);
            const int r = KC ? r0 + line : r0 + off;
            const int k = KC ? k0 + off : k0 + line;
            const bool ok = r < rmax && k < kmax;
            const bf16_t* src = KC ? g + (int64_t)r * ld + k : g + (int64_t)k * ld + r;
            if constexpr (VEC == 8) {
                uint4 x = make_uint4(0u, 0u, 0u, 0u);
                if (ok) x = *reinterpret_cast<const uint4*>(src);
                v[4 * i + 0] = x.x;
                v[4 * i + 1] = x.y;
                v[4 * i + 2] = x.z;
                v[4 * i + 3] = x.w;
            } else {
                v[i] = ok ? (uint32_t)*src : 0u;
            }
        }
    }

    __device__ __forceinline__ void store(bf16_t* s, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int line, off;
            where(tid, i, line, off);
            if constexpr (VEC == 8)
                *reinterpret_cast<uint4*>(s + line * LD + off) =
                    make_uint4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
            else
                s[line * LD + off] = (bf16_t)v[i];
        }
    }

    // Eight k-values (16c + 8*(lane/32) + 0..7) of tile row base + lane%32.
    __device__ __forceinline__ static bf16x8v read(const bf16_t* s, int base, int c, int lane) {
        const int kb = 16 * c + 8 * (lane >> 5);
        if constexpr (KC) {
            return *reinterpret_cast<const bf16x8v*>(s + (base + (lane & 31)) * LD + kb);
        } else {
            const int sl = lane & 15;
            const int col = base + 16 * ((lane >> 4) & 1) + 4 * (sl & 3);
            const bf16_t* p0 = s + (kb + (sl >> 2)) * LD + col;
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p0);
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p0 + 4 * LD));
            const short8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            return __builtin_bit_cast(bf16x8v, both);
        }
    }
};


template <class S, Layout LAY, int VEC, Epi EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_kernel(GemmParams p) {
    constexpr int BM = S::BM, BN = S::BN, FM = S::FM, FN = S::FN;
    using TA = Tile<BM, LAY != Layout::TN, VEC>;
    using TB = Tile<BN, LAY == Layout::NT, VEC>;
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][TA::ELEMS];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][TB::ELEMS];
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
    TA la;
    TB lb;

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
#pragma unroll
            for (int c = 0; c < kBK / 16; ++c) {
                bf16x8v a[FM], b[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) a[i] = TA::read(sA[cur], wm * S::WM + 32 * i, c, lane);
#pragma unroll
                for (int j = 0; j < FN; ++j) b[j] = TB::read(sB[cur], wn * S::WN + 32 * j, c, lane);
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
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float16v sum;
#pragma unroll
                for (int r = 0; r < 16; ++r) sum[r] = 0.f;
                for (int t = 0; t < p.splits; ++t) {
                    const float* q = p.partials + (int64_t)t * p.M * p.N;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = row_w + i * 32 + 8 * (r >> 2) + (r & 3);
                        const int col = col_w + j * 32;
                        float v = acc[i][j][r];
                        if (t != split && row < p.M && col < p.N)
                            v = load_coherent(q + (int64_t)row * p.N + col);
                        sum[r] += v;
                    }
                }
                acc[i][j] = sum;
            }
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

template <class S, Layout LAY, Epi EPI>
hipError_t go_vec(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    return L.vec == 8 ? go<S, LAY, 8, EPI>(p, L.grid, st) : go<S, LAY, 1, EPI>(p, L.grid, st);
}

template <class S>
hipError_t dispatch_shape(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    switch (L.layout) {
    case Layout::NN:
        if (L.epi == Epi::ReluMask) return go_vec<S, Layout::NN, Epi::ReluMask>(L, p, st);
        if (L.epi == Epi::Store) return go_vec<S, Layout::NN, Epi::Store>(L, p, st);
        break;
    case Layout::NT:
        if (L.epi == Epi::MaskMul) return go_vec<S, Layout::NT, Epi::MaskMul>(L, p, st);
        break;
    case Layout::TN:
        if (L.epi == Epi::Sgd) return go_vec<S, Layout::TN, Epi::Sgd>(L, p, st);
        if (L.epi == Epi::Adapt) return go_vec<S, Layout::TN, Epi::Adapt>(L, p, st);
        if (L.epi == Epi::Grad) return go_vec<S, Layout::TN, Epi::Grad>(L, p, st);
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
    default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace mlp
