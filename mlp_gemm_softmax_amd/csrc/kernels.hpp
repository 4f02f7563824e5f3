// Host-visible launch interface of the step's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace mlp {

// Operand layouts of C[M,N] = A[M,K] . B[K,N] (row-major storage):
//   NN: A stored [M][K], B stored [K][N]   forward  a_{l-1} . W_l
//   NT: A stored [M][K], B stored [N][K]   dX       G_l . W_l^T
//   TN: A stored [K][M], B stored [K][N]   dW       a_{l-1}^T . G_l
enum class Layout : int { NN = 0, NT = 1, TN = 2 };

// Fused epilogues applied to the float32 accumulator v at (row, col):
//   Store    C = v                                  (logits)
//   ReluMask C = max(v, 0) (f32 or bf16), mask = v > 0
//   MaskMul  C = mask ? v : 0 (f32 or bf16)        (dX through the ReLU)
//   Sgd      W = W - lr * v, optional bf16 copy    (dW + in-place update)
//   Grad     C = v                                  (dW, no update)
//   Adapt    W, m, v <- Adam or LaProp step with g = v (optional bf16 copy)
enum class Epi : int { Store = 0, ReluMask = 1, MaskMul = 2, Sgd = 3, Grad = 4, Adapt = 5, Softmax = 6 };

// Scalars of an adaptive update step (Adam or LaProp, see optim_rule.hpp).
constexpr int kOptAdam = 1;
constexpr int kOptLaProp = 2;
struct OptScalars {
    int rule;                              // kOptAdam or kOptLaProp
    float lr, b1, b2, om1, om2, eps;       // om = 1 - beta
    float inv_c1, inv_c2;                  // 1 / (1 - beta^t)
};

struct GemmParams {
    const void* A;       // float or bf16, per the kernel's precision
    const void* B;
    int64_t lda, ldb;
    int M, N, K;
    float* C;            // f32 output, or the f32 master W for Sgd
    bf16_t* Cb;          // bf16 output (ReluMask/MaskMul in bf16 mode, Sgd shadow)
    uint8_t* mask;       // ReluMask writes, MaskMul reads; [M][N], leading dim ldc
    int64_t ldc;
    float lr;
    int splits;          // K split into `splits` chunks of `kchunk`
    int kchunk;
    float* partials;     // [splits][M][N] float32 when splits > 1
    unsigned* tickets;   // one zeroed counter per output tile when splits > 1
    int tiles_m, tiles_n;
    float* m;            // Adapt: first and second moments, laid out as C
    float* v;
    OptScalars opt;      // Adapt: the step's scalars
};

// Tile configurations of the MFMA GEMM (workgroup tile BM x BN, 4 waves).
// T256x256 is the large-tile kernel (direct-to-LDS loads, bf16 or f32 operands).
// T32x32 / T32x16 are the small-product kernel's tiles (one per workgroup).
enum class TileCfg : int { T128x128 = 0, T64x64 = 1, T32x128 = 2, T128x32 = 3, T128x64 = 4,
                           T256x256 = 5, T32x32 = 6, T32x16 = 7 };
void tile_shape(TileCfg cfg, int* bm, int* bn);

struct GemmLaunch {
    Layout layout;
    Epi epi;
    bool bf16;       // bf16 operands (MLP_BF16) or f32 operands
    TileCfg cfg;
    int vec;         // 4 (or 8 for bf16) if k-contiguous operands allow wide loads, else 1
    int grid;        // workgroups
};

hipError_t launch_gemm(const GemmLaunch& L, const GemmParams& p, hipStream_t s);

// Large-tile kernel (bf16 or f32 operands, L.bf16): whether its 16-byte
// direct loads suit the operands, its one-time set-up, and the launch.
bool gemm_big_fits(bool bf16, Layout lay, int M, int N, int K, int64_t lda, int64_t ldb);
hipError_t gemm_big_prepare();
// With reduce = false a split product (Store epilogue only) leaves its sums
// in p.partials for a later launch (launch_splitk_xent) to add.
hipError_t launch_gemm_big(const GemmLaunch& L, const GemmParams& p, hipStream_t s, bool reduce = true);
// Adds the K splits' partials [splits][M][N] in split order and applies the
// epilogue (used by the large-tile kernel when it splits K).
hipError_t launch_splitk_epilogue(const GemmParams& p, Epi epi, hipStream_t s);

// Small float32 products: one 32x32 (L.cfg == T32x32) or 32x16 (T32x16)
// tile per workgroup, K split across its `waves` waves and reduced in LDS (no
// split-K across workgroups).  Uses L.layout, L.epi, L.vec, L.cfg and
// L.grid = ceil(M/32) * ceil(N/32 or 16).
int gemm_small_waves(int M, int N, int K);
hipError_t launch_gemm_small(const GemmLaunch& L, const GemmParams& p, int waves, hipStream_t s);

// ---- skinny batch (B <= 16) float32 kernels ------------------------------
struct SkinnyParams {
    const float* A;   // NN: x [MB][K] ; NT: W [Kout][N] ; TN: a [MB][K]
    const float* B;   // NN: W [K][N]  ; NT: G [MB][N]   ; TN: G [MB][N]
    int MB;           // batch rows
    int K, N;         // NN: out [MB][N] = x.W ; NT: out [MB][Kout=K] ; TN: W [K][N]
    float* C;         // output / W master
    bf16_t* Cb;
    uint8_t* mask;
    float lr;
    int splits, kchunk;
    float* partials;
    unsigned* tickets;
    const float* act;  // NT with fused update: a [MB][K] of the layer's input
    float* wout;       // NT with fused update: W (Sgd/Adapt, in place) or dW (Grad)
    float* m;          // Adapt: first and second moments, laid out as W
    float* v;
    OptScalars opt;    // Adapt: the step's scalars
    const float* grad; // NN with fused update: G [MB][N] of the previous step (act: its input a)
    // NT with fused update: with loss set, wavefront 0 of workgroup 0 also
    // writes the mean of the MB row losses, which the softmax-CE launch
    // before it left undone (XentParams::defer_mean); MB <= 64
    const float* rowloss = nullptr;
    float* loss = nullptr;
    float inv_b = 0.f;
};
struct SkinnyLaunch {
    Layout layout;
    Epi epi;
    int grid;
    int waves;       // waves per workgroup
    bool fused_update = false;   // NT: also apply the layer's dW (+ SGD) in the same pass;
                                 // NN: first apply the previous step's dW + SGD to W (act, grad, wout = W)
};
hipError_t launch_skinny(const SkinnyLaunch& L, const SkinnyParams& p, hipStream_t s);
int skinny_tn_rows();   // rows of W per dW+SGD workgroup

// ---- class probabilities (inference) -----------------------------------
// probs[b][c] = exp(z[b][c] - max_c z[b]) / sum_c exp(z[b][c] - max_c z[b]),
// one wavefront per row, fixed-order wavefront reductions.
hipError_t launch_softmax_rows(const float* logits, float* probs, int B, int C, hipStream_t st);

// ---- softmax cross-entropy -------------------------------------------------
struct XentParams {
    const float* logits;   // [B][C]
    const float* labels;   // [B][C]
    float* dlogits;        // [B][C] f32
    bf16_t* dlogits_b;     // [B][C] bf16 copy or null
    float* rowloss;        // [B]
    float* loss;           // scalar mean loss
    unsigned* ticket;      // zeroed counter
    int B, C;
    float inv_b;
    bool defer_mean = false;   // write the row losses only; the next launch takes their mean
};
hipError_t launch_xent(const XentParams& p, int* grid_out, hipStream_t s);
// Split-K sum of the logits product's partials [splits][B][C] (split order),
// logits store and softmax-CE in one launch; C % 4 == 0, C <= 1024, 2..4 splits.
bool splitk_xent_fits(int C, int splits);
hipError_t launch_splitk_xent(const XentParams& p, const float* partials, int splits, float* logits,
                              hipStream_t s);

// ---- fused output layer for C <= 32 (logits, softmax-CE, dX) --------------
struct HeadParams {
    const float* A;        // a_{L-1} [B][H]
    const float* W;        // W_L [H][C] (read; updated later by the tail)
    const float* labels;   // [B][C]
    const uint8_t* mask;   // m_{L-1} [B][H]
    float* logits;         // [B][C] or null
    float* dlogits;        // [B][C]
    float* G;              // dZ_{L-1} [B][H]
    float* rowloss;        // [B]
    int B, H, C, CP, RB;   // CP = C | 1 (LDS row stride of W), RB rows per workgroup
    float inv_b;
};
size_t head_lds_bytes(int H, int C, int RB);
int head_max_lds();          // dynamic LDS the head kernel may use
hipError_t head_prepare();   // raise the kernel's dynamic-LDS limit once
hipError_t launch_head(const HeadParams& p, hipStream_t s);

// ---- tail of the fused output layer: dW_L (+ SGD) and the mean loss ------
// Runs after the head, either as extra workgroups of the last small-product
// launch of the step (gemm_small, T32x16) or on its own.  Job j < ceil(H/16)
// owns rows 16j..16j+15 of dW_L (K = B on the matrix core, no cross-
// workgroup reduction); job ceil(H/16) adds the row losses.
struct TailParams {
    const float* A;        // a_{L-1} [B][H]
    const float* dZ;       // dlogits [B][C]
    float* W;              // W_L [H][C], updated in place unless dW is set
    float* dW;             // gradient output or null
    const float* rowloss;  // [B]
    float* loss;           // scalar mean loss
    int B, H, C;
    float lr, inv_b;
    float* m;              // non-null (and dW null): Adam / LaProp moments of W_L
    float* v;
    OptScalars opt;
};
__host__ __device__ inline int tail_jobs(int H) { return (H + 15) / 16 + 1; }
hipError_t launch_tail(const TailParams& t, hipStream_t s);
// The last hidden layer's small-product forward (32 x 16 tiles, 16 waves)
// with the head run by the workgroup finishing each 32-row block (hp.RB =
// 32; p.tickets: one zeroed counter per row block).
hipError_t launch_gemm_small_head(const GemmLaunch& L, const GemmParams& p, const HeadParams& hp, hipStream_t s);
// The last small-product dW launch with the tail's jobs as extra workgroups.
hipError_t launch_gemm_small_tail(const GemmLaunch& L, const GemmParams& p, int waves, const TailParams& t,
                                  hipStream_t s);

// ---- f32 -> bf16 cast -----------------------------------------------------
hipError_t launch_cast_bf16(const float* src, bf16_t* dst, size_t n, hipStream_t s);

// ---- optimizer state (optim.hip) --------------------------------------------
// Zero n floats (n % 4 == 0, 16-byte aligned) with a kernel.
hipError_t launch_zero(float* p, size_t n, hipStream_t s);
// ---- bf16 -> f32 widen (state read-back) -----------------------------------
hipError_t launch_widen_bf16(const bf16_t* src, float* dst, size_t n, hipStream_t s);

}  // namespace mlp
