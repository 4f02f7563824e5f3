// MFMA GEMM with 256 x 256 workgroup tiles for the large products of both
// contracts: bfloat16 operands (v_mfma_f32_32x32x16_bf16, 64-deep k stages)
// or float32 operands (v_mfma_f32_32x32x2f32, 32-deep stages), float32
// accumulate, the step's fused epilogues; with the K split in up to 4 parts
// the partial sums go to memory and a separate all-CU kernel adds them and
// applies the epilogue.  A stage is 128 bytes of k per tile row in both
// precisions, so the LDS geometry below is shared; where the text says
// "element" it is 2 bytes (bf16) or 4 (f32).
//
// Why a second kernel: at 128 x 128 tiles the LDS traffic per MFMA flop
// (fragment reads plus tile writes) exceeds what one CU's LDS delivers while
// the matrix cores run at full rate, and the L2 -> CU operand traffic per
// flop is twice that of a 256 x 256 tile.  Here
//   - 4 waves, each owning a 128 x 128 sub-tile (16 accumulators of 32 x 32,
//     v_mfma_f32_32x32x16_bf16), so every LDS fragment feeds 4 MFMAs;
//   - operands go from global memory into LDS 16 bytes per lane, either
//     straight (buffer_load_dwordx4 ... lds) or through registers
//     (buffer_load_dwordx4, then ds_write_b128 into the same place before the
//     next barrier); the results are the same bit for bit.  Direct loads are
//     faster for bf16 NT (both operands read with ds_read_b128), staging
//     through registers for the layouts with transpose reads and for f32
//     (measured 3-11% and about 1%).  Lanes whose element lies outside the
//     matrix get an offset past the buffer's size, which the hardware turns
//     into zeros;
//   - two k stages (2 x 64 KB of LDS, four static arrays): the loads
//     of stage k+1 are in flight while stage k is multiplied; one barrier per
//     stage;
//   - bank-conflict-free layouts by XOR swizzles (the direct loads write 1 KB
//     contiguous per wave instruction, so rows cannot be padded):
//       k-contiguous operand: LDS row r (128 B of k) holds 16-byte chunk j
//         of the global row at chunk slot j ^ ((r >> 1) & 7); an MFMA operand
//         is one ds_read_b128 per lane (8 bf16 or 4 f32 k-values);
//       r-contiguous operand, bf16: LDS k-row (512 B = 256 r) holds the
//         64-byte segment s (32 r) at slot s ^ (k & 3); an MFMA operand is
//         two ds_read_b64_tr_b16 per lane (transpose reads, as in the
//         128-wide kernel), the four k-rows one read touches landing in
//         distinct banks;
//       r-contiguous operand, f32: LDS k-row (1 KB = 256 r) in global order;
//         an operand is four ds_read_b32 per lane (k, k+1, k+2, k+3), each
//         half-wave reading 32 consecutive floats.
//   - float32: one ds_read_b128 of the k-contiguous operand holds 4 k-values,
//     and MFMA q (0..3) of a chunk takes value q: lanes 0-31 supply
//     k = 8c + q and lanes 32-63 k = 8c + 4 + q, the same map for both
//     operands, so the four MFMAs of a chunk add up all 8 k-values.
#include "epilogue4.hpp"
#include <type_traits>

#include "kernels.hpp"

namespace mlp {
namespace {

constexpr int kT = 256;                  // tile rows and columns
constexpr int kThreads = 256;            // 4 waves, 2 x 2, 128 x 128 each
constexpr int kOpBytes = 32 * 1024;      // one operand tile per stage: 256 rows x 128 bytes of k

// Per-precision constants: k per stage, bytes per element, the MFMA operand.
template <bool F32>
struct Elem {
    static constexpr int kBK = F32 ? 32 : 64;
    static constexpr int ES = F32 ? 4 : 2;
    using Frag = typename std::conditional<F32, float4v, bf16x8v>::type;
};
constexpr unsigned kOob = 0x80000000u;   // buffer offset that reads as zero
constexpr int kMaxSplits = 4;            // K splits the reduction handles

typedef short short4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) void lds_void;

// Per-lane source offsets of one operand tile's 8 direct-load instructions
// (this wave's share of 32 KB), relative to the tile's first k.
template <bool KC, bool F32>
struct Loader {
    unsigned off[8];   // element offset of the row (KC) or column (MN) part, or kOob outside the matrix
    int kk[8];         // k of this lane's chunk within the stage

    __device__ __forceinline__ void init(int64_t ld, int r0, int rmax, int wave, int lane) {
        constexpr int VE = 16 / Elem<F32>::ES;   // elements per 16-byte chunk
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = wave * 8 + i;
            if constexpr (KC) {
                const int r = 8 * q + (lane >> 3);
                const int j = (lane & 7) ^ ((r >> 1) & 7);
                kk[i] = VE * j;
                off[i] = r0 + r < rmax ? (unsigned)((int64_t)(r0 + r) * ld) : kOob;
            } else if constexpr (F32) {
                // one k-row of 256 floats per instruction, in global order
                kk[i] = q;
                off[i] = r0 + 4 * lane < rmax ? (unsigned)(r0 + 4 * lane) : kOob;
            } else {
                const int k = 2 * q + (lane >> 5);
                const int p = lane & 31;
                const int col = (((p >> 2) ^ (k & 3)) << 5) + 8 * (p & 3);
                kk[i] = k;
                off[i] = r0 + col < rmax ? (unsigned)(r0 + col) : kOob;
            }
        }
    }

    // Byte offset of load i of stage k0, or kOob.
    __device__ __forceinline__ unsigned src(int i, int64_t ld, int k0, int kmax) const {
        const int k = k0 + kk[i];
        if (off[i] == kOob || k >= kmax) return kOob;
        return (unsigned)Elem<F32>::ES * (KC ? off[i] + (unsigned)k : (unsigned)((int64_t)k * ld) + off[i]);
    }

    // Register staging: load stage k0 into r, later write r where the direct
    // loads would have put it.
    __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int kmax,
                                          u32x4v (&r)[8]) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)src(i, ld, k0, kmax), 0, 0);
    }
    __device__ __forceinline__ static void commit(char* dst, int wave, int lane, const u32x4v (&r)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4v*>(dst + (wave * 8 + i) * 1024 + lane * 16) = r[i];
    }

    // Issue the 8 loads of stage k0 into `dst` (this operand's 32 KB tile).
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t ld, int k0, int kmax,
                                          char* dst, int wave) const {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (wave * 8 + i) * 1024), 16,
                                                     src(i, ld, k0, kmax), 0, 0, 0);
    }
};

// The k-values of chunk c for tile row `base` + lane%32: bf16, eight
// (16c + 8*(lane/32) + 0..7); f32, four (8c + 4*(lane/32) + 0..3).
template <bool KC, bool F32>
__device__ __forceinline__ typename Elem<F32>::Frag frag(const char* s, int base, int c, int lane) {
    using Frag = typename Elem<F32>::Frag;
    if constexpr (KC) {
        const int r = base + (lane & 31);
        const int j = (2 * c + (lane >> 5)) ^ ((r >> 1) & 7);
        return *reinterpret_cast<const Frag*>(s + r * 128 + j * 16);
    } else if constexpr (F32) {
        const int k = 8 * c + 4 * (lane >> 5);
        const float* p = reinterpret_cast<const float*>(s) + k * kT + base + (lane & 31);
        float4v v;
        v[0] = p[0];
        v[1] = p[kT];
        v[2] = p[2 * kT];
        v[3] = p[3 * kT];
        return v;
    } else {
        const int sl = lane & 15;
        const int k = 16 * c + 8 * (lane >> 5) + (sl >> 2);
        const int seg = (base >> 5) ^ (k & 3);
        const char* p0 = s + k * 512 + seg * 64 + 32 * ((lane >> 4) & 1) + 8 * (sl & 3);
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)p0);
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p0 + 4 * 512));
        const short8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8v, both);
    }
}

// Bytes from the first element to one past the last of a row-major matrix
// with `rows` rows of `cols` used elements and leading dimension ld.
template <bool F32>
__device__ __forceinline__ unsigned extent_bytes(int rows, int cols, int64_t ld) {
    return (unsigned)(Elem<F32>::ES * ((int64_t)(rows - 1) * ld + cols));
}

// The MFMAs of one chunk for accumulator block (i, j).
template <bool F32>
__device__ __forceinline__ float16v mfma_chunk(const typename Elem<F32>::Frag& a, const typename Elem<F32>::Frag& b,
                                               float16v acc) {
    if constexpr (F32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
        return acc;
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
}

// One k stage on LDS buffer (ca, cb); (na, nb) holds the next stage.
// Chunks 0-2 multiply while the following chunk's fragments are read; then,
// once this thread's loads of the next stage have landed and every wave has
// passed the barrier, the loads of the stage after next go out into the
// buffer just finished, and chunk 3 multiplies while chunk 0 of the next
// stage is read.  The buffers are distinct LDS arrays known at compile time,
// so the compiler's wait counting sees that reads of one buffer do not depend
// on the direct loads in flight into the other.  With register staging (REG)
// the stage after next is loaded into (pa, pb) instead, and those registers,
// loaded during the previous stage, are written into (na, nb) during chunks
// 1 (A) and 2 (B), before the barrier that makes them visible.
template <bool AKC, bool BKC, bool F32, bool REG>
__device__ __forceinline__ void stage(float16v (&acc)[4][4], typename Elem<F32>::Frag (&a)[2][4],
                                      typename Elem<F32>::Frag (&b)[2][4], char* ca, char* cb, char* na,
                                      char* nb, const Loader<AKC, F32>& la, const Loader<BKC, F32>& lb,
                                      u32x4v (&pa)[8], u32x4v (&pb)[8],
                                      __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                      const GemmParams& p, int kload, int kend, int wm, int wn,
                                      int wave, int lane) {
    // f32: 64 MFMAs per chunk and up to 32 LDS reads (four per r-contiguous
    // operand); one read after every second MFMA, one direct load after
    // every fourth in the last chunk
    constexpr int ND = 4 * (AKC ? 1 : 4) + 4 * (BKC ? 1 : 4);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const int f = c & 1;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[f ^ 1][i] = frag<AKC, F32>(ca, wm * 128 + 32 * i, c + 1, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[f ^ 1][j] = frag<BKC, F32>(cb, wn * 128 + 32 * j, c + 1, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_chunk<F32>(a[f][i], b[f][j], acc[i][j]);
        // constant once the loop is unrolled: A's staged writes in chunk 1,
        // B's in chunk 2
        const bool kCommit = REG && (c == 1 || c == 2);
        if (REG && c == 1) Loader<AKC, F32>::commit(na, wave, lane, pa);
        if (REG && c == 2) Loader<BKC, F32>::commit(nb, wave, lane, pb);
        if constexpr (F32) {
#pragma unroll
            for (int u = 0; u < 64; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (u % 2 == 0 && u / 2 < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (kCommit && u % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
        } else {
            // one fragment read (and in chunks 1-2 one staged write) after each MFMA
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (kCommit) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!REG) wait_loads();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) a[0][i] = frag<AKC, F32>(na, wm * 128 + 32 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[0][j] = frag<BKC, F32>(nb, wn * 128 + 32 * j, 0, lane);
    if constexpr (REG) {
        la.fetch(ra, p.lda, kload, kend, pa);
        lb.fetch(rb, p.ldb, kload, kend, pb);
    } else {
        la.issue(ra, p.lda, kload, kend, ca, wave);
        lb.issue(rb, p.ldb, kload, kend, cb, wave);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_chunk<F32>(a[1][i], b[1][j], acc[i][j]);
    if constexpr (F32) {
#pragma unroll
        for (int u = 0; u < 64; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (u % 2 == 0 && u / 2 < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (u % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    } else {
        // one fragment read and one direct load after each of the first 12
        // MFMAs, the remaining loads after the last 4 (the reads target the
        // other buffer, which the compiler's wait counting tells apart)
#pragma unroll
        for (int u = 0; u < 12; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <bool F32, Layout LAY, Epi EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_big_kernel(GemmParams p) {
    constexpr bool AKC = LAY != Layout::TN;   // A stored [M][K]
    constexpr bool BKC = LAY == Layout::NT;   // B stored [N][K]
    constexpr bool kReg = F32 || LAY != Layout::NT;   // register staging (see the header)
    constexpr int kBK = Elem<F32>::kBK;
    using Frag = typename Elem<F32>::Frag;
    __shared__ __attribute__((aligned(16))) char sa0[kOpBytes], sb0[kOpBytes], sa1[kOpBytes], sb1[kOpBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // Split-major order: the workgroups that share an XCD (consecutive ids)
    // work on the same k range of neighbouring tiles and share operands in L2.
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
    const int m0 = tm * kT, n0 = tn * kT;
    const int kbeg = split * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = kend > kbeg ? (kend - kbeg + kBK - 1) / kBK : 0;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(p.A), (short)0,
        AKC ? extent_bytes<F32>(p.M, p.K, p.lda) : extent_bytes<F32>(p.K, p.M, p.lda),
        0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(p.B), (short)0,
        BKC ? extent_bytes<F32>(p.N, p.K, p.ldb) : extent_bytes<F32>(p.K, p.N, p.ldb),
        0x00020000);
    Loader<AKC, F32> la;
    Loader<BKC, F32> lb;
    la.init(p.lda, m0, p.M, wave, lane);
    lb.init(p.ldb, n0, p.N, wave, lane);

    float16v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
        // Stage t lives in buffer t & 1; stages past the end load as zeros
        // and are never multiplied.
        u32x4v pa[8], pb[8];
        if constexpr (kReg) {
            // stage 0 written now, stage 1 held in registers until the
            // first stage writes it
            la.fetch(ra, p.lda, kbeg, kend, pa);
            lb.fetch(rb, p.ldb, kbeg, kend, pb);
            Loader<AKC, F32>::commit(sa0, wave, lane, pa);
            Loader<BKC, F32>::commit(sb0, wave, lane, pb);
            la.fetch(ra, p.lda, kbeg + kBK, kend, pa);
            lb.fetch(rb, p.ldb, kbeg + kBK, kend, pb);
            __syncthreads();
        } else {
            la.issue(ra, p.lda, kbeg, kend, sa0, wave);
            lb.issue(rb, p.ldb, kbeg, kend, sb0, wave);
            wait_loads();
            __syncthreads();
            la.issue(ra, p.lda, kbeg + kBK, kend, sa1, wave);
            lb.issue(rb, p.ldb, kbeg + kBK, kend, sb1, wave);
        }
        Frag a[2][4], b[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[0][i] = frag<AKC, F32>(sa0, wm * 128 + 32 * i, 0, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[0][j] = frag<BKC, F32>(sb0, wn * 128 + 32 * j, 0, lane);
        // Stages in pairs (buffer 0, buffer 1); an odd count multiplies one
        // all-zero stage at the end, which adds exact zeros.
        for (int kt = 0; kt < nk; kt += 2) {
            stage<AKC, BKC, F32, kReg>(acc, a, b, sa0, sb0, sa1, sb1, la, lb, pa, pb, ra, rb, p,
                                       kbeg + (kt + 2) * kBK, kend, wm, wn, wave, lane);
            stage<AKC, BKC, F32, kReg>(acc, a, b, sa1, sb1, sa0, sb0, la, lb, pa, pb, ra, rb, p,
                                       kbeg + (kt + 3) * kBK, kend, wm, wn, wave, lane);
        }
        // the zero-filling direct loads of the stages past the end (staged
        // loads of those stages land in registers that are never read)
        if constexpr (!kReg) wait_loads();
    }

    // Epilogue.  Each wave stages its 128 x 128 accumulators through LDS, 32
    // rows at a time (row stride 132 floats), and reads them back row-major:
    // lane l takes float4 q of row 2q + l/32, columns 4(l%32)..+3, so every
    // global access is a coalesced 16-byte (f32) or 8-byte (bf16) vector.
    // The mask bytes of all four chunks (64 registers) are requested before
    // the staging starts, so their latency is paid once; the SGD weights
    // (256 registers for all chunks) are read chunk by chunk.
    const int rbase = m0 + wm * 128 + (lane >> 5);
    const int col = n0 + wn * 128 + 4 * (lane & 31);
    constexpr bool kAllPre = EPI == Epi::MaskMul;
    Pre pre[kAllPre ? 4 : 1][EPI == Epi::Adapt ? 1 : 16];   // Adapt reads its inputs per quarter chunk
    if (kAllPre && p.splits == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (rbase + 32 * i + 2 * q < p.M && col < p.N)
                    pre[i][q] = epilogue_load<EPI>(p, rbase + 32 * i + 2 * q, col);
    }
    __syncthreads();   // every wave is done with the stage buffers
    float* st = reinterpret_cast<float*>(wave == 0 ? sa0 : wave == 1 ? sb0 : wave == 2 ? sa1 : sb1);
    constexpr int SP = 132;
    // one 32-row chunk; the chunk index is a template constant so that the
    // accumulators are indexed statically (a loop the compiler declines to
    // unroll would put them in scratch memory)
    auto chunk = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                st[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SP + 32 * j + (lane & 31)] = acc[i][j][r];
        float4v v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
            v[q] = *reinterpret_cast<const float4v*>(st + (2 * q + (lane >> 5)) * SP + 4 * (lane & 31));
        const int row0 = rbase + 32 * i;
        if (p.splits > 1) {
            // K split: this split's sums go to partials [split][M][N]; the
            // split-K epilogue kernel adds them in split order
            float* part = p.partials + (int64_t)split * p.M * p.N;
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (row0 + 2 * q < p.M && col < p.N)
                    *reinterpret_cast<float4v*>(part + (int64_t)(row0 + 2 * q) * p.N + col) = v[q];
            return;
        }
        if constexpr (EPI == Epi::Adapt) {
            // W, m and v of 16 rows would not fit the registers: 4 at a time
#pragma unroll
            for (int hq = 0; hq < 16; hq += 4) {
                Pre ph[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (row0 + 2 * (hq + q) < p.M && col < p.N) ph[q] = epilogue_load<EPI>(p, row0 + 2 * (hq + q), col);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (row0 + 2 * (hq + q) < p.M && col < p.N)
                        epilogue4<EPI>(p, row0 + 2 * (hq + q), col, v[hq + q], ph[q]);
            }
        } else {
            Pre* pr = pre[kAllPre ? i : 0];
            if constexpr (!kAllPre) {
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (row0 + 2 * q < p.M && col < p.N) pr[q] = epilogue_load<EPI>(p, row0 + 2 * q, col);
            }
#pragma unroll
            for (int q = 0; q < 16; ++q)
                if (row0 + 2 * q < p.M && col < p.N) epilogue4<EPI>(p, row0 + 2 * q, col, v[q], pr[q]);
        }
        };
    chunk(std::integral_constant<int, 0>{});
    chunk(std::integral_constant<int, 1>{});
    chunk(std::integral_constant<int, 2>{});
    chunk(std::integral_constant<int, 3>{});

}

template <bool F32, Layout LAY, Epi EPI>
hipError_t go(const GemmParams& p, int grid, bool reduce, hipStream_t st) {
    hipLaunchKernelGGL((gemm_big_kernel<F32, LAY, EPI>), dim3(grid), dim3(kThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.splits > 1 && reduce) e = launch_splitk_epilogue(p, EPI, st);
    return e;
}

template <bool F32>
hipError_t dispatch(const GemmLaunch& L, const GemmParams& p, hipStream_t st, bool reduce) {
    switch (L.layout) {
    case Layout::NN:
        if (L.epi == Epi::ReluMask) return go<F32, Layout::NN, Epi::ReluMask>(p, L.grid, reduce, st);
        if (L.epi == Epi::Store) return go<F32, Layout::NN, Epi::Store>(p, L.grid, reduce, st);
        break;
    case Layout::NT:
        if (L.epi == Epi::MaskMul) return go<F32, Layout::NT, Epi::MaskMul>(p, L.grid, reduce, st);
        break;
    case Layout::TN:
        if (L.epi == Epi::Sgd) return go<F32, Layout::TN, Epi::Sgd>(p, L.grid, reduce, st);
        if (L.epi == Epi::Adapt) return go<F32, Layout::TN, Epi::Adapt>(p, L.grid, reduce, st);
        if (L.epi == Epi::Grad) return go<F32, Layout::TN, Epi::Grad>(p, L.grid, reduce, st);
        break;
    }
    return hipErrorInvalidValue;
}


}  // namespace

bool gemm_big_fits(bool bf16, Layout lay, int M, int N, int K, int64_t lda, int64_t ldb) {
    // 16-byte direct loads: contiguous extents and leading dimensions in
    // whole 16-byte chunks; buffer offsets below 2^31 bytes.
    const int ve = bf16 ? 8 : 4, es = bf16 ? 2 : 4;
    const bool akc = lay != Layout::TN, bkc = lay == Layout::NT;
    const int acont = akc ? K : M, bcont = bkc ? K : N;
    if (acont % ve || bcont % ve || lda % ve || ldb % ve) return false;
    const int64_t arows = akc ? M : K, brows = bkc ? N : K;
    return es * arows * lda < (int64_t)kOob && es * brows * ldb < (int64_t)kOob;
}

hipError_t gemm_big_prepare() { return hipSuccess; }

hipError_t launch_gemm_big(const GemmLaunch& L, const GemmParams& p, hipStream_t st, bool reduce) {
    if (p.splits < 1 || p.splits > kMaxSplits || L.grid != p.tiles_m * p.tiles_n * p.splits)
        return hipErrorInvalidValue;
    // without the reduction only the raw partials of a split product are
    // written; its epilogue must then be Store (the caller reduces them)
    if (!reduce && p.splits > 1 && L.epi != Epi::Store) return hipErrorInvalidValue;
    // float32 sessions keep no bfloat16 copies
    if (!L.bf16 && p.Cb) return hipErrorInvalidValue;
    return L.bf16 ? dispatch<false>(L, p, st, reduce) : dispatch<true>(L, p, st, reduce);
}

}  // namespace mlp
