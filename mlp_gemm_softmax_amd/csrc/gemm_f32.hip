// Strict-float32 MFMA GEMM for the step's three products (forward NN, dX NT,
// dW TN) with fused epilogues, LDS double buffering and deterministic
// split-K.  The matmul archetype of the Meganeura README ("Why Meganeura":
// shaders composed from pointwise, reduction and matmul archetypes) on
// gfx950 matrix cores: v_mfma_f32_32x32x2f32, 64 flop/clk per SIMD.
//
// Workgroup: 256 threads = 4 wavefronts, tile BM x BN, K staged 32 at a time.
// Each operand tile keeps its global orientation in LDS, so global->LDS is a
// straight 16-byte copy whichever way the operand is stored:
//   k-contiguous operand (row r, k):  LDS [r][k], row stride 36 floats;
//   r-contiguous operand (k, row r):  LDS [k][r], row stride R+4 floats.
// For an MFMA both supply the same k map: over a chunk of 8 k, lanes 0-31
// hold k = 8c..8c+3 and lanes 32-63 hold k = 8c+4..8c+7 of row lane%32, and
// MFMA q (q = 0..3) takes the q-th of those four values.  A k-contiguous tile
// delivers the four values in one 16-byte LDS read, an r-contiguous tile in
// four 4-byte reads (consecutive lanes -> consecutive banks).
#include "kernels.hpp"
#include "epilogue1.hpp"

namespace mlp {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;

template <int BM_, int BN_, int WM_, int WN_>
struct Shape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int WAVES_N = BN / WN;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
};

// Operand tile of R rows x kBK k.  KC: stored k-contiguous (element (r,k) at
// g + r*ld + k), else r-contiguous (at g + k*ld + r).  VEC: 4 = 16-byte global
// loads (the contiguous extent and ld are multiples of 4), 1 = 4-byte loads.
template <int R, bool KC, int VEC>
struct Tile {
    static constexpr int LD = KC ? kBK + 4 : R + 4;          // LDS row stride (floats)
    static constexpr int ELEMS = KC ? R * LD : kBK * LD;     // LDS floats per stage
    static constexpr int CONT = KC ? kBK : R;                // contiguous extent per line
    static constexpr int PER = R * kBK / (kThreads * VEC);   // global accesses per thread
    static_assert(PER >= 1, "tile too small for the loader");
    float v[PER * VEC];

    // (line, offset) of access i: a line is a k-row (r-contiguous) or an r-row.
    __device__ __forceinline__ static void where(int tid, int i, int& line, int& off) {
        const int idx = tid + kThreads * i;
        line = idx / (CONT / VEC);
        off = (idx % (CONT / VEC)) * VEC;
    }

    __device__ __forceinline__ void load(const float* __restrict__ g, int64_t ld, int r0, int rmax,
                                         int k0, int kmax, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int line, off;
            where(tid, i, line, off);
            const int r = KC ? r0 + line : r0 + off;
            const int k = KC ? k0 + off : k0 + line;
            const bool ok = r < rmax && k < kmax;
            const float* src = KC ? g + (int64_t)r * ld + k : g + (int64_t)k * ld + r;
            if constexpr (VEC == 4) {
                float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
                if (ok) x = *reinterpret_cast<const float4*>(src);
                v[4 * i + 0] = x.x;
                v[4 * i + 1] = x.y;
                v[4 * i + 2] = x.z;
                v[4 * i + 3] = x.w;
            } else {
                v[i] = ok ? *src : 0.f;
            }
        }
    }

    __device__ __forceinline__ void store(float* s, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            int line, off;
            where(tid, i, line, off);
            if constexpr (VEC == 4)
                *reinterpret_cast<float4*>(s + line * LD + off) =
                    make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
            else
                s[line * LD + off] = v[i];
        }
    }

    // The four k-values of MFMA chunk c for tile row `row`, lane half h.
    __device__ __forceinline__ static float4v read(const float* s, int row, int c, int h) {
        const int k = 8 * c + 4 * h;
        if constexpr (KC) {
            return *reinterpret_cast<const float4v*>(s + row * LD + k);
        } else {
            float4v r;
            r[0] = s[(k + 0) * LD + row];
            r[1] = s[(k + 1) * LD + row];
            r[2] = s[(k + 2) * LD + row];
            r[3] = s[(k + 3) * LD + row];
            return r;
        }
    }
};


template <class S, Layout LAY, int VEC, Epi EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_f32_kernel(GemmParams p) {
    constexpr int BM = S::BM, BN = S::BN, FM = S::FM, FN = S::FN;
    using TA = Tile<BM, LAY != Layout::TN, VEC>;
    using TB = Tile<BN, LAY == Layout::NT, VEC>;
    __shared__ __attribute__((aligned(16))) float sA[2][TA::ELEMS];
    __shared__ __attribute__((aligned(16))) float sB[2][TB::ELEMS];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

    // Logical workgroup id -> (split, output tile); tiles are visited in
    // groups of 8 tile-rows so concurrently running tiles share operands.
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

    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    float16v acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int arow = wm * S::WM + (lane & 31);
    const int brow = wn * S::WN + (lane & 31);
    const int half = lane >> 5;

    auto compute = [&](const float* a_s, const float* b_s) {
#pragma unroll
        for (int c = 0; c < kBK / 8; ++c) {
            float4v a[FM], b[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) a[i] = TA::read(a_s, arow + 32 * i, c, half);
#pragma unroll
            for (int j = 0; j < FN; ++j) b[j] = TB::read(b_s, brow + 32 * j, c, half);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][q], b[j][q], acc[i][j], 0, 0, 0);
        }
    };

    TA la;
    TB lb;
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
            compute(sA[cur], sB[cur]);
            if (more) {
                la.store(sA[cur ^ 1], tid);
                lb.store(sB[cur ^ 1], tid);
            }
            __syncthreads();
        }
    }

    // Accumulator element r of block (i, j) sits at
    //   row = 8*(r/4) + 4*(lane/32) + r%4,  col = lane%32   within the block.
    const int row_w = m0 + wm * S::WM + 4 * half;
    const int col_w = n0 + wn * S::WN + (lane & 31);

    if (p.splits > 1) {
        // Deterministic split-K: every split stores its partial tile; the
        // workgroup that takes the last ticket sums the partials in split
        // order 0..S-1 and applies the epilogue.
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
        // One 32x32 block at a time; the loads of TU splits are in flight
        // together, then added in split order.
        constexpr int TU = FM * FN >= 4 ? 1 : 4 / (FM * FN);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                float16v sum;
#pragma unroll
                for (int r = 0; r < 16; ++r) sum[r] = 0.f;
                for (int t0 = 0; t0 < p.splits; t0 += TU) {
                    float16v v[TU];
#pragma unroll
                    for (int u = 0; u < TU; ++u) {
                        const int t = t0 + u;
                        const float* q = p.partials + (int64_t)t * p.M * p.N;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int row = row_w + i * 32 + 8 * (r >> 2) + (r & 3);
                            const int col = col_w + j * 32;
                            float x = 0.f;
                            if (t == split) x = acc[i][j][r];
                            else if (t < p.splits && row < p.M && col < p.N)
                                x = load_coherent(q + (int64_t)row * p.N + col);
                            v[u][r] = x;
                        }
                    }
#pragma unroll
                    for (int u = 0; u < TU; ++u) sum += v[u];
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
    hipLaunchKernelGGL((gemm_f32_kernel<S, LAY, VEC, EPI>), dim3(grid), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <class S, Layout LAY, Epi EPI>
hipError_t go_vec(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    return L.vec == 4 ? go<S, LAY, 4, EPI>(p, L.grid, st) : go<S, LAY, 1, EPI>(p, L.grid, st);
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

hipError_t launch_gemm_f32(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
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
