// Step engine and C ABI of libmlp.so (declared in include/mlp.h).
//
// mlp_create plans one static graph: it carves the caller's workspace into
// fixed buffers (weights, bf16 operand copies, activations, masks, logits,
// dlogits, a ping-pong pair of dZ buffers, split-K partials and integer
// tickets) and picks a tile shape and K split for every product.  A training
// step is then a fixed launch sequence on one stream:
//
//   [bf16: cast x]
//   for l = 0..L-2:  NN  a_{l+1}, m_{l+1} = relu(a_l W_l)        (ReluMask)
//                    NN  logits = a_{L-1} W_{L-1}                (Store)
//                    softmax-CE -> dlogits, row losses, mean loss
//   for l = L-1..0:  NT  G_l = (G_{l+1} W_l^T) * m_l  if l > 0   (MaskMul)
//                    TN  W_l -= lr * a_l^T G_{l+1}               (Sgd)
//
// The dX product of a layer is enqueued before its dW+SGD product, which
// overwrites the weights it reads (the step's gradients are all taken at the
// pre-update weights).  With B <= 16 in float32 the three products use the
// skinny-batch streaming kernels instead of the tiled MFMA GEMM.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mlp.h"
#include "kernels.hpp"

namespace mlp {
hipError_t launch_gemm_f32(const GemmLaunch& L, const GemmParams& p, hipStream_t st);
hipError_t launch_gemm_bf16(const GemmLaunch& L, const GemmParams& p, hipStream_t st);

hipError_t launch_gemm(const GemmLaunch& L, const GemmParams& p, hipStream_t st) {
    if (L.cfg == TileCfg::T256x256) return launch_gemm_big(L, p, st);
    return L.bf16 ? launch_gemm_bf16(L, p, st) : launch_gemm_f32(L, p, st);
}

void tile_shape(TileCfg cfg, int* bm, int* bn) {
    switch (cfg) {
    case TileCfg::T128x128: *bm = 128; *bn = 128; return;
    case TileCfg::T64x64: *bm = 64; *bn = 64; return;
    case TileCfg::T32x128: *bm = 32; *bn = 128; return;
    case TileCfg::T128x32: *bm = 128; *bn = 32; return;
    case TileCfg::T128x64: *bm = 128; *bn = 64; return;
    case TileCfg::T256x256: *bm = 256; *bn = 256; return;
    case TileCfg::T32x32: *bm = 32; *bn = 32; return;
    case TileCfg::T32x16: *bm = 32; *bn = 16; return;
    }
    *bm = *bn = 0;
}
}  // namespace mlp

using namespace mlp;

namespace {

constexpr int kMaxLayers = 16;
constexpr int kMaxDim = 1 << 20;
constexpr int kSkinnyMaxBatch = 16;
constexpr size_t kAlign = 256;
constexpr size_t kGuardBytes = 256;       // least guard band after a workspace buffer
constexpr unsigned char kGuardByte = 0xA5;

thread_local std::string g_create_error;

struct GemmPlan {
    TileCfg cfg = TileCfg::T128x128;
    int splits = 1, kchunk = 0, tiles_m = 1, tiles_n = 1, grid = 1;
    int vec = 1;
    int small_waves = 0;    // > 0: the small-product kernel with this many waves
};

struct SkinnyPlan {
    int grid = 1, waves = 4, splits = 1, kchunk = 0, tickets = 0;
};

struct Slot {
    std::string name;
    double flops = 0, bytes = 0;
    double total_ms = 0;
    int64_t launches = 0;
};

struct Pending {
    int kind, slot;
    hipEvent_t beg, end;
};

// Launch sequences that are timed separately: a training step (or
// gradients), a forward pass, a forward pass with the loss, a forward pass
// to class probabilities.
enum SlotKind { kStep = 0, kForward = 1, kForwardLoss = 2, kForwardProbs = 3, kKinds = 4 };

}  // namespace

struct mlp_ctx {
    int L = 0;
    int dims[kMaxLayers + 1] = {};
    int B = 0;
    bool bf16 = false;
    bool skinny = false;
    bool head = false;      // fused output layer (C <= 32, f32)
    bool external_w = false;   // weights are the caller's (no workspace room for them)
    int head_rb = 0;        // batch rows per head workgroup
    hipStream_t stream = nullptr;

    // workspace buffers
    float* W[kMaxLayers] = {};
    bf16_t* Wb[kMaxLayers] = {};
    void* act[kMaxLayers] = {};        // a_l, l = 1..L-1 (f32 or bf16)
    uint8_t* mask[kMaxLayers] = {};    // m_l, l = 1..L-1
    bf16_t* xb = nullptr;
    float* logits = nullptr;
    float* dlogits = nullptr;
    bf16_t* dlogits_b = nullptr;
    void* dz[2] = {};
    float* partials = nullptr;
    unsigned* tickets = nullptr;
    size_t partial_cap = 0, ticket_cap = 0;   // elements / counters the plans may use
    unsigned* xent_ticket = nullptr;
    float* rowloss = nullptr;
    float* loss_slot = nullptr;

    GemmPlan fwd[kMaxLayers], dx[kMaxLayers], dw[kMaxLayers];
    SkinnyPlan sfwd[kMaxLayers], sdx[kMaxLayers], sdw[kMaxLayers];

    unsigned params_set = 0;   // bit l: W_l written since creation / poisoning
    bool poisoned = false;
    std::string err;
    std::string failed_launch;   // slot of the launch whose HIP call failed, if any

    // Guard bands: a run of kGuardByte after every sub-buffer of the
    // workspace (from the buffer's last byte to the next buffer), filled at
    // creation and compared on the host when MLP_DEBUG_GUARDS is set.
    struct Guard {
        std::string after;   // buffer the band follows
        size_t off, len;     // byte range in the workspace
    };
    std::vector<Guard> guards;
    char* base = nullptr;
    unsigned debug = 0;        // MLP_DEBUG_* flags

    // update rule of a training step: SGD (no state), or Adam / LaProp with
    // moments in caller memory given to mlp_set_optimizer, applied by the dW
    // launches while they hold W
    int opt = MLP_OPT_SGD;
    float opt_b1 = 0.f, opt_b2 = 0.f, opt_eps = 0.f;
    int64_t opt_t = 0;                  // steps taken with the current moments
    float* opt_m[kMaxLayers] = {};
    float* opt_v[kMaxLayers] = {};

    bool profiling = false;
    std::vector<Slot> slots[kKinds];   // per launch sequence
    int prof_kind = kStep;             // sequence of the last call enqueued while profiling
    std::vector<Pending> pending;
    std::vector<hipEvent_t> event_pool;
};

namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

mlp_status set_err(mlp_ctx* c, mlp_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (c) c->err = buf; else g_create_error = buf;
    return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------------ plans --

GemmPlan plan_gemm(int M, int N, int K, bool bf16, bool kvec_ok, bool big_ok) {
    GemmPlan g;
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (big_ok) {
        // Large products: 256 x 256 tiles, one workgroup per CU; K is split
        // (up to 4 ways, at least 512 deep) while the tiles fill fewer than
        // half the CUs.
        const int nt = tiles(256, 256);
        const int sk = bf16 ? 64 : 32;   // k per stage
        int s = 1;
        if (nt < 128) s = std::max(1, std::min({4, (256 + nt - 1) / nt, K / 512}));
        if (nt * s >= 128) {
            int kchunk = (K + s - 1) / s;
            kchunk = (kchunk + sk - 1) / sk * sk;
            s = (K + kchunk - 1) / kchunk;
            g.cfg = TileCfg::T256x256;
            g.tiles_m = (M + 255) / 256;
            g.tiles_n = (N + 255) / 256;
            g.splits = s;
            g.kchunk = s > 1 ? kchunk : std::max(K, 1);
            g.grid = nt * s;
            g.vec = bf16 ? 8 : 4;
            return g;
        }
    }
    if (M <= 32) g.cfg = TileCfg::T32x128;
    else if (N <= 32) g.cfg = TileCfg::T128x32;
    else if (tiles(128, 128) >= 240) g.cfg = TileCfg::T128x128;
    else if (tiles(128, 64) >= 240) g.cfg = TileCfg::T128x64;
    else g.cfg = TileCfg::T64x64;
    int bm, bn;
    tile_shape(g.cfg, &bm, &bn);
    g.tiles_m = (M + bm - 1) / bm;
    g.tiles_n = (N + bn - 1) / bn;
    const int nt = g.tiles_m * g.tiles_n;
    const int bk = bf16 ? 64 : 32;
    const int t32 = ((M + 31) / 32) * ((N + 31) / 32);
    if (!bf16 && nt < 256 && t32 <= 1024) {
        // Under-filled product: K split inside the workgroup, no partials;
        // 32 x 16 tiles while 32 x 32 ones would leave CUs idle.
        g.small_waves = gemm_small_waves(M, N, K);
        g.splits = 1;
        g.kchunk = std::max(K, 1);
        const int t16 = ((M + 31) / 32) * ((N + 15) / 16);
        g.cfg = t32 < 256 ? TileCfg::T32x16 : TileCfg::T32x32;
        g.grid = t32 < 256 ? t16 : t32;
        g.vec = kvec_ok ? 4 : 1;
        return g;
    }
    const int target = 512;
    const int kmin = bf16 ? 256 : 128;
    int s = std::max(1, std::min((target + nt - 1) / nt, K / kmin));
    int kchunk = (K + s - 1) / s;
    kchunk = (kchunk + bk - 1) / bk * bk;
    s = (K + kchunk - 1) / kchunk;
    g.splits = std::max(1, s);
    g.kchunk = g.splits > 1 ? kchunk : std::max(K, 1);
    g.grid = nt * g.splits;
    g.vec = kvec_ok ? (bf16 ? 8 : 4) : 1;
    return g;
}

// Split-K partial floats a plan needs: [splits][M][N], or whole padded tiles
// for the large-tile kernel.
size_t partial_elems(const GemmPlan& g, int M, int N) {
    if (g.splits <= 1) return 0;
    if (g.cfg == TileCfg::T256x256) return (size_t)g.splits * g.tiles_m * 256 * g.tiles_n * 256;
    return (size_t)g.splits * M * N;
}

SkinnyPlan plan_skinny_nn(int N, int K, int B) {
    (void)B;
    SkinnyPlan s;
    // 64 output columns per workgroup of 8 waves; K splits only while the
    // grid still fits one round of workgroups (measured at batch 8: 16-wave
    // workgroups and deeper splits stream slower).
    const int ncg = (N + 63) / 64;
    s.waves = 8;
    int sp = std::max(1, std::min(256 / ncg, K / 256));
    int kchunk = (K + sp - 1) / sp;
    kchunk = (kchunk + 15) / 16 * 16;
    sp = (K + kchunk - 1) / kchunk;
    s.splits = sp;
    s.kchunk = sp > 1 ? kchunk : K;
    s.grid = ncg * sp;
    s.tickets = ncg;
    return s;
}

double es(bool bf16) { return bf16 ? 2.0 : 4.0; }

// Whether the fused output layer's tail can ride along with the first
// layer's dW launch (the 32 x 16 small-product kernel), else it runs alone.
bool tail_fused(const mlp_ctx* c) {
    return c->head && !c->skinny && c->dw[0].small_waves > 0 && c->dw[0].cfg == TileCfg::T32x16;
}

// Whether the last hidden layer's forward plan could carry the output
// layer's head (32 x 16 small-product tiles with 16 waves; the workgroup
// finishing a 32-row block runs the head for it).
bool head_fusable(const mlp_ctx* c) {
    if (!c->head || c->skinny || c->L < 2) return false;
    const GemmPlan& g = c->fwd[c->L - 2];
    return g.small_waves == 16 && g.cfg == TileCfg::T32x16 &&
           head_lds_bytes(c->dims[c->L - 1], c->dims[c->L], 32) <= 64 * 1024;
}

// Whether the head runs inside that launch, which takes one ticket per
// 32-row block; else the head runs in a launch of its own.
bool head_fused(const mlp_ctx* c) {
    return head_fusable(c) && (size_t)(c->B + 31) / 32 <= c->ticket_cap;
}

OptScalars opt_scalars(const mlp_ctx* c, float lr) {
    OptScalars o{};
    o.rule = c->opt == MLP_OPT_ADAM ? kOptAdam : kOptLaProp;
    o.lr = lr;
    o.b1 = c->opt_b1;
    o.b2 = c->opt_b2;
    o.om1 = (float)(1.0 - (double)c->opt_b1);
    o.om2 = (float)(1.0 - (double)c->opt_b2);
    o.eps = c->opt_eps;
    o.inv_c1 = (float)(1.0 / (1.0 - std::pow((double)c->opt_b1, (double)c->opt_t)));
    o.inv_c2 = (float)(1.0 / (1.0 - std::pow((double)c->opt_b2, (double)c->opt_t)));
    return o;
}

// Whether the softmax-CE launch also adds the split-K partials of the logits
// product (large-tile bf16 forward split over K): the logits are then written
// once, by the loss kernel, and not read back.
bool xent_fused(const mlp_ctx* c) {
    if (c->head || c->skinny) return false;
    const GemmPlan& g = c->fwd[c->L - 1];
    return g.cfg == TileCfg::T256x256 && g.splits > 1 && splitk_xent_fits(c->dims[c->L], g.splits);
}

// Whether a forward pass to probabilities normalises inside the logits
// product (f32 small-product kernel, every class in one 16-column tile),
// else a row-softmax launch follows the product.
bool probs_fused(const mlp_ctx* c) {
    const GemmPlan& g = c->fwd[c->L - 1];
    return !c->bf16 && !c->skinny && g.small_waves > 0 && g.cfg == TileCfg::T32x16 && c->dims[c->L] <= 16;
}

// Slot names and algorithmic work of one launch sequence, in launch order.
void build_slot_list(mlp_ctx* c, int sk) {
    std::vector<Slot>& slots = c->slots[sk];
    slots.clear();
    const int L = c->L, B = c->B;
    const double e = es(c->bf16);
    auto add = [&](const std::string& n, double f, double b) {
        Slot s;
        s.name = n;
        s.flops = f;
        s.bytes = b;
        slots.push_back(s);
    };
    // a forward call runs the output layer as plain products, never the head
    const bool head = c->head && sk == kStep;
    const char* kind = c->skinny ? "skinny" : (c->bf16 ? "mfma_bf16" : "mfma_f32");
    // with an adaptive rule the dW launches store gradients and one more
    // launch applies the update
    // the update every dW launch applies while it holds W
    const std::string upd = c->opt == MLP_OPT_SGD ? "sgd" : (c->opt == MLP_OPT_ADAM ? "adam" : "laprop");
    const double mv = c->opt == MLP_OPT_SGD ? 0.0 : 16.0;   // m and v in and out, per weight
    if (c->bf16) add("cast_x_bf16", 0, (double)B * c->dims[0] * 6);
    const int C = c->dims[L];
    const int Lf = head ? L - 1 : L;   // layers whose forward is a plain GEMM
    const bool xf = xent_fused(c) && (sk == kStep || sk == kForwardLoss);   // the loss launch adds the logits' partials
    const bool pf = sk == kForwardProbs && probs_fused(c);
    for (int l = 0; l < Lf; ++l) {
        const double M = B, N = c->dims[l + 1], K = c->dims[l];
        const bool last = l == L - 1;
        // a product that leaves its split-K sums to the loss kernel has no
        // compulsory output of its own
        const double out = last ? (xf ? 0.0 : M * N * 4) : M * N * (e + 1);
        const char* what = last ? (xf ? "partials" : (pf ? "softmax" : "store")) : "relu_mask";
        add(std::string(kind) + "_nn_" + what + "_l" + std::to_string(l), 2 * M * N * K, M * K * e + K * N * e + out);
    }
    if (sk == kForward) return;
    if (sk == kForwardProbs) {
        if (!pf) add("softmax_probs", 0, (double)B * C * 8);   // logits in, probabilities out
        return;
    }
    int top = L - 1;
    double tail_flops = 0, tail_bytes = 0;
    std::string tail_name;
    if (head) {
        const double H = c->dims[L - 1];
        const std::string hn = "head_logits_xent_dx_l" + std::to_string(L - 1);
        const double hf = 4.0 * B * H * C, hb = B * H * 4 + H * C * 4 + B * C * 12 + B * H * 5 + B * 4.0;
        if (head_fused(c)) {   // merge into the last hidden layer's forward slot
            Slot& f = slots.back();
            f.name += "+" + hn;
            f.flops += hf;
            f.bytes += hb;
        } else {
            add(hn, hf, hb);
        }
        top = L - 2;
        tail_flops = 2.0 * B * H * C;
        tail_bytes = B * H * 4 + B * C * 4 + H * C * (8 + mv) + B * 4.0;
        tail_name = "tail_dw_" + upd + "_loss_l" + std::to_string(L - 1);
    } else {
        if (xf)   // labels in; logits, dlogits (+ bf16 copy) and row losses out
            add("splitk_sum_softmax_xent", 0, (double)B * C * (12 + (c->bf16 ? 2 : 0)) + B * 4.0);
        else      // logits and labels in; dlogits (+ bf16 copy) and row losses out
            add("softmax_xent", 0, (double)B * C * (12 + (c->bf16 ? 2 : 0)) + B * 4.0);
    }
    if (sk == kForwardLoss) return;
    for (int l = top; l >= 0; --l) {
        const double din = c->dims[l], dout = c->dims[l + 1];
        if (l > 0 && c->skinny) {
            // dX and dW + update in one pass over W: W read and written once
            // (with an adaptive rule m and v too)
            add(std::string(kind) + "_nt_mask_" + upd + "_l" + std::to_string(l), 4.0 * B * din * dout,
                (8.0 + mv) * din * dout + 4.0 * B * dout + 4.0 * B * din + B * din * 5.0);
            continue;
        }
        if (l > 0)
            add(std::string(kind) + "_nt_mask_l" + std::to_string(l), 2.0 * B * din * dout,
                B * dout * e + din * dout * e + B * din * (1 + e));
        // W in+out (+ bf16 copy), and m, v in+out with an adaptive rule
        const double wb = 8 + (c->bf16 ? 2 : 0) + mv;
        const double f = 2.0 * B * din * dout, b = B * din * e + B * dout * e + din * dout * wb;
        if (l == 0 && head && tail_fused(c))
            add(std::string(kind) + "_tn_" + upd + "_l0+" + tail_name, f + tail_flops, b + tail_bytes);
        else
            add(std::string(kind) + "_tn_" + upd + "_l" + std::to_string(l), f, b);
    }
    if (head && !tail_fused(c)) add(tail_name, tail_flops, tail_bytes);
}

void build_slots(mlp_ctx* c) {
    for (int k = 0; k < kKinds; ++k) build_slot_list(c, k);
}

// ---------------------------------------------------------------- launches --

bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

struct Runner {
    mlp_ctx* c;
    int kind = kStep;
    bool off = false;   // no per-launch timing for this sequence
    hipError_t err = hipSuccess;

    hipEvent_t ev() {
        if (!c->event_pool.empty()) {
            hipEvent_t e = c->event_pool.back();
            c->event_pool.pop_back();
            return e;
        }
        // device-scope release: a default event's system-scope release
        // writes the L2 back around every launch, which would be timed too
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventReleaseToDevice) != hipSuccess) return nullptr;
        return e;
    }

    template <class F>
    void run(int slot_id, F&& f) {
        if (err != hipSuccess) return;
        hipEvent_t b = nullptr, e = nullptr;
        if (c->profiling && !off && slot_id >= 0) {
            b = ev();
            e = ev();
            if (b && e) hipEventRecord(b, c->stream);
        }
        err = f();
        if (b && e) {
            hipEventRecord(e, c->stream);
            c->pending.push_back({kind, slot_id, b, e});
        }
        // Serial mode: wait for each launch so that a failure that shows only
        // at execution is charged to the launch that caused it.
        if (err == hipSuccess && (c->debug & MLP_DEBUG_SYNC) && !capturing(c->stream))
            err = hipStreamSynchronize(c->stream);
        if (err != hipSuccess) {
            if (slot_id >= 0 && slot_id < (int)c->slots[kind].size())
                c->failed_launch = c->slots[kind][slot_id].name;
            else
                c->failed_launch = "launch " + std::to_string(slot_id);
        }
    }
};

hipError_t run_gemm(mlp_ctx* c, const GemmPlan& g, Layout lay, Epi epi, const void* A, int64_t lda,
                    const void* Bm, int64_t ldb, int M, int N, int K, float* C, bf16_t* Cb,
                    uint8_t* mask, float lr, const TailParams* tail = nullptr, bool reduce = true,
                    float* m = nullptr, float* v = nullptr, const OptScalars* opt = nullptr) {
    GemmLaunch L;
    L.layout = lay;
    L.epi = epi;
    L.bf16 = c->bf16;
    L.cfg = g.cfg;
    L.vec = g.vec;
    L.grid = g.grid;
    GemmParams p;
    p.A = A;
    p.B = Bm;
    p.lda = lda;
    p.ldb = ldb;
    p.M = M;
    p.N = N;
    p.K = K;
    p.C = C;
    p.Cb = Cb;
    p.mask = mask;
    p.ldc = N;
    p.lr = lr;
    p.splits = g.splits;
    p.kchunk = g.kchunk;
    p.partials = c->partials;
    p.tickets = c->tickets;
    p.tiles_m = g.tiles_m;
    p.tiles_n = g.tiles_n;
    p.m = m;
    p.v = v;
    p.opt = opt ? *opt : OptScalars{};
    if (tail) return launch_gemm_small_tail(L, p, g.small_waves, *tail, c->stream);
    if (g.small_waves > 0) return launch_gemm_small(L, p, g.small_waves, c->stream);
    if (g.cfg == TileCfg::T256x256) return launch_gemm_big(L, p, c->stream, reduce);
    return launch_gemm(L, p, c->stream);
}


hipError_t run_skinny(mlp_ctx* c, const SkinnyPlan& s, Layout lay, Epi epi, const float* A,
                      const float* Bm, int K, int N, float* C, uint8_t* mask, float lr,
                      float* m = nullptr, float* v = nullptr, const OptScalars* opt = nullptr) {
    SkinnyLaunch L;
    L.layout = lay;
    L.epi = epi;
    L.grid = s.grid;
    L.waves = s.waves;
    SkinnyParams p;
    p.A = A;
    p.B = Bm;
    p.MB = c->B;
    p.K = K;
    p.N = N;
    p.C = C;
    p.Cb = nullptr;
    p.mask = mask;
    p.lr = lr;
    p.splits = s.splits;
    p.kchunk = s.kchunk;
    p.partials = c->partials;
    p.tickets = c->tickets;
    p.act = nullptr;
    p.wout = nullptr;
    p.m = m;
    p.v = v;
    p.opt = opt ? *opt : OptScalars{};
    p.grad = nullptr;
    return launch_skinny(L, p, c->stream);
}

// Whether a run of training steps can hand the first layer's dW + SGD of one
// step to the next step's first forward launch: skinny float32 sessions with
// plain SGD and at most 8 batch rows.
bool steps_fusable(const mlp_ctx* c) {
    return c->skinny && !c->bf16 && c->opt == MLP_OPT_SGD && c->B <= 8;
}


enum class Mode { Forward, Train, Grads };

// Enqueue the step.  Returns the first HIP error (launches stop there).
// Within a run of steps (mlp_train_steps, skinny sessions): with x_next the
// first layer's dW + SGD launch also computes the next step's first forward
// on x_next, and first_done says this step's first forward was made that way.
hipError_t enqueue(mlp_ctx* c, Mode mode, const float* x, const float* labels, float lr,
                   float* const* dw_out, float* loss_dev, float* probs = nullptr,
                   bool first_done = false, const float* x_next = nullptr) {
    Runner r{c, mode != Mode::Forward ? kStep : (probs ? kForwardProbs : (labels ? kForwardLoss : kForward))};
    // the per-launch timing names the single-step launch sequence
    r.off = first_done || x_next;
    if (c->profiling && !r.off) c->prof_kind = r.kind;
    const int L = c->L, B = c->B;
    int slot = 0;
    const void* a_prev;
    if (c->bf16) {
        r.run(slot++, [&] { return launch_cast_bf16(x, c->xb, (size_t)B * c->dims[0], c->stream); });
        a_prev = c->xb;
    } else {
        a_prev = x;
    }
    // ---- forward (with the fused head the last layer's matmul is in the head)
    const bool use_head = c->head && mode != Mode::Forward;
    const bool fuse_head = use_head && head_fused(c);
    const int C = c->dims[L];
    auto head_params = [&](int RB) {
        HeadParams hp;
        hp.A = (const float*)c->act[L - 1];
        hp.W = c->W[L - 1];
        hp.labels = labels;
        hp.mask = c->mask[L - 1];
        hp.logits = c->logits;
        hp.dlogits = c->dlogits;
        hp.G = (float*)c->dz[0];
        hp.rowloss = c->rowloss;
        hp.B = B;
        hp.H = c->dims[L - 1];
        hp.C = C;
        hp.CP = C | 1;
        hp.RB = RB;
        hp.inv_b = 1.0f / (float)B;
        return hp;
    };
    for (int l = 0; l < (use_head ? L - 1 : L); ++l) {
        const int K = c->dims[l], N = c->dims[l + 1];
        const bool last = l == L - 1;
        const void* Wop = c->bf16 ? (const void*)c->Wb[l] : (const void*)c->W[l];
        if (c->skinny && l == 0 && first_done) {
            // made by the previous step's first-layer update launch
        } else if (c->skinny) {
            r.run(slot++, [&] {
                return run_skinny(c, c->sfwd[l], Layout::NN, last ? Epi::Store : Epi::ReluMask,
                                  (const float*)a_prev, (const float*)Wop, K, N,
                                  last ? c->logits : (float*)c->act[l + 1],
                                  last ? nullptr : c->mask[l + 1], 0.f);
            });
        } else if (fuse_head && l == L - 2) {
            r.run(slot++, [&] {
                const GemmPlan& g = c->fwd[l];
                GemmLaunch gl;
                gl.layout = Layout::NN;
                gl.epi = Epi::ReluMask;
                gl.bf16 = false;
                gl.cfg = g.cfg;
                gl.vec = g.vec;
                gl.grid = g.grid;
                GemmParams gp{};
                gp.A = a_prev;
                gp.B = Wop;
                gp.lda = K;
                gp.ldb = N;
                gp.M = B;
                gp.N = N;
                gp.K = K;
                gp.C = (float*)c->act[l + 1];
                gp.mask = c->mask[l + 1];
                gp.ldc = N;
                gp.splits = 1;
                gp.kchunk = K;
                gp.tickets = c->tickets;
                return launch_gemm_small_head(gl, gp, head_params(32), c->stream);
            });
        } else {
            // with labels the loss kernel adds a split logits product's partials
            const bool partials_only = last && labels && xent_fused(c);
            const bool to_probs = last && probs && probs_fused(c);
            r.run(slot++, [&] {
                if (to_probs)
                    return run_gemm(c, c->fwd[l], Layout::NN, Epi::Softmax, a_prev, K, Wop, N, B, N, K, probs,
                                    nullptr, nullptr, 0.f);
                float* Cf = last ? c->logits : (c->bf16 ? nullptr : (float*)c->act[l + 1]);
                bf16_t* Cb = (!last && c->bf16) ? (bf16_t*)c->act[l + 1] : nullptr;
                return run_gemm(c, c->fwd[l], Layout::NN, last ? Epi::Store : Epi::ReluMask, a_prev, K,
                                Wop, N, B, N, K, Cf, Cb, last ? nullptr : c->mask[l + 1], 0.f, nullptr,
                                !partials_only);
            });
        }
        if (!last) a_prev = c->act[l + 1];
    }
    if (mode == Mode::Forward && probs) {
        if (!probs_fused(c)) r.run(slot++, [&] { return launch_softmax_rows(c->logits, probs, B, C, c->stream); });
        return r.err;
    }
    if (mode == Mode::Forward && !labels) return r.err;

    // ---- loss
    // In skinny sessions with a hidden layer the launch after the softmax-CE
    // is the last layer's fused dX + dW pass; it takes the mean of the row
    // losses, so the softmax-CE launch ends without its ticketed mean.
    const bool defer_mean = c->skinny && !use_head && L >= 2 && B <= 64 && mode != Mode::Forward;
    if (use_head) {
        if (!fuse_head) r.run(slot++, [&] { return launch_head(head_params(c->head_rb), c->stream); });
    } else {
        r.run(slot++, [&] {
            XentParams xp;
            xp.logits = c->logits;
            xp.labels = labels;
            xp.dlogits = c->dlogits;
            xp.dlogits_b = c->bf16 ? c->dlogits_b : nullptr;
            xp.rowloss = c->rowloss;
            xp.loss = loss_dev ? loss_dev : c->loss_slot;
            xp.ticket = c->xent_ticket;
            xp.B = B;
            xp.C = C;
            xp.inv_b = 1.0f / (float)B;
            xp.defer_mean = defer_mean;
            if (xent_fused(c)) return launch_splitk_xent(xp, c->partials, c->fwd[L - 1].splits, c->logits, c->stream);
            return launch_xent(xp, nullptr, c->stream);
        });
    }
    if (mode == Mode::Forward) return r.err;

    // ---- backward (every dW launch applies the update while it holds W)
    const bool adaptive = mode == Mode::Train && c->opt != MLP_OPT_SGD;
    const bool grads = mode == Mode::Grads;
    const Epi upd_epi = grads ? Epi::Grad : (adaptive ? Epi::Adapt : Epi::Sgd);
    const OptScalars osc = adaptive ? opt_scalars(c, lr) : OptScalars{};
    TailParams tp{};
    if (use_head) {
        tp.A = (const float*)c->act[L - 1];
        tp.dZ = c->dlogits;
        tp.W = c->W[L - 1];
        tp.dW = grads ? dw_out[L - 1] : nullptr;
        tp.m = adaptive ? c->opt_m[L - 1] : nullptr;
        tp.v = adaptive ? c->opt_v[L - 1] : nullptr;
        tp.opt = osc;
        tp.rowloss = c->rowloss;
        tp.loss = loss_dev ? loss_dev : c->loss_slot;
        tp.B = B;
        tp.H = c->dims[L - 1];
        tp.C = C;
        tp.lr = lr;
        tp.inv_b = 1.0f / (float)B;
    }
    const bool fuse_tail = use_head && tail_fused(c);
    // The separate tail reads a_{L-1}, which a first-layer launch that also
    // makes the next step's forward overwrites when L = 2: it needs only the
    // head's outputs, so then it goes first.
    const bool tail_early = use_head && !fuse_tail && x_next;
    if (tail_early) r.run(slot++, [&] { return launch_tail(tp, c->stream); });
    const void* G = c->bf16 ? (const void*)c->dlogits_b : (const void*)c->dlogits;
    int pp = 0;
    int top = L - 1;
    if (use_head) {           // the head produced G_{L-1} in dz[0] and updated W_{L-1}
        G = c->dz[0];
        pp = 1;
        top = L - 2;
    }
    for (int l = top; l >= 0; --l) {
        const int din = c->dims[l], dout = c->dims[l + 1];
        const void* Wop = c->bf16 ? (const void*)c->Wb[l] : (const void*)c->W[l];
        const void* Gnext = nullptr;
        if (l > 0 && c->skinny) {
            // one pass over W_l: G_{l-1} (from the old W_l) and the update
            void* out = c->dz[pp];
            pp ^= 1;
            r.run(slot++, [&] {
                SkinnyLaunch sl;
                sl.layout = Layout::NT;
                sl.epi = upd_epi;
                sl.grid = c->sdx[l].grid;
                sl.waves = 8;
                sl.fused_update = true;
                SkinnyParams sp{};
                sp.A = c->W[l];
                sp.B = (const float*)G;
                sp.MB = B;
                sp.K = din;
                sp.N = dout;
                sp.C = (float*)out;
                sp.mask = c->mask[l];
                sp.lr = lr;
                sp.act = (const float*)c->act[l];
                sp.wout = grads ? dw_out[l] : c->W[l];
                sp.m = adaptive ? c->opt_m[l] : nullptr;
                sp.v = adaptive ? c->opt_v[l] : nullptr;
                sp.opt = osc;
                sp.splits = c->sdx[l].splits;
                sp.kchunk = c->sdx[l].kchunk;
                sp.partials = c->partials;
                sp.tickets = c->tickets;
                if (defer_mean && l == L - 1) {
                    sp.rowloss = c->rowloss;
                    sp.loss = loss_dev ? loss_dev : c->loss_slot;
                    sp.inv_b = 1.0f / (float)B;
                }
                return launch_skinny(sl, sp, c->stream);
            });
            G = out;
            continue;
        }
        if (l > 0) {
            void* out = c->dz[pp];
            pp ^= 1;
            r.run(slot++, [&] {
                return run_gemm(c, c->dx[l], Layout::NT, Epi::MaskMul, G, dout, Wop, dout, B, din, dout,
                                c->bf16 ? nullptr : (float*)out, c->bf16 ? (bf16_t*)out : nullptr, c->mask[l],
                                0.f);
            });
            Gnext = out;
        }
        const void* a_in = l == 0 ? (c->bf16 ? (const void*)c->xb : (const void*)x) : c->act[l];
        float* Wdst = grads ? dw_out[l] : c->W[l];
        bf16_t* Wbdst = (!grads && c->bf16) ? c->Wb[l] : nullptr;
        float* om = adaptive ? c->opt_m[l] : nullptr;
        float* ov = adaptive ? c->opt_v[l] : nullptr;
        if (c->skinny && l == 0 && x_next) {
            // this step's dW + SGD of W_0, then the next step's forward of
            // layer 0 on x_next with the updated W_0, in one pass over W_0
            r.run(slot++, [&] {
                const SkinnyPlan& sf = c->sfwd[0];
                const bool only = L == 1;
                SkinnyLaunch sl;
                sl.layout = Layout::NN;
                sl.epi = only ? Epi::Store : Epi::ReluMask;
                sl.grid = sf.grid;
                sl.waves = sf.waves;
                sl.fused_update = true;
                SkinnyParams sp{};
                sp.A = x_next;
                sp.B = c->W[0];
                sp.MB = B;
                sp.K = din;
                sp.N = dout;
                sp.C = only ? c->logits : (float*)c->act[1];
                sp.mask = only ? nullptr : c->mask[1];
                sp.lr = lr;
                sp.splits = sf.splits;
                sp.kchunk = sf.kchunk;
                sp.partials = c->partials;
                sp.tickets = c->tickets;
                sp.act = x;
                sp.grad = (const float*)G;
                sp.wout = c->W[0];
                return launch_skinny(sl, sp, c->stream);
            });
        } else if (c->skinny) {
            r.run(slot++, [&] {
                return run_skinny(c, c->sdw[l], Layout::TN, upd_epi, (const float*)a_in, (const float*)G, din, dout,
                                  Wdst, nullptr, lr, om, ov, &osc);
            });
        } else {
            r.run(slot++, [&] {
                return run_gemm(c, c->dw[l], Layout::TN, upd_epi, a_in, din, G, dout, din, dout, B, Wdst, Wbdst,
                                nullptr, lr, (l == 0 && fuse_tail) ? &tp : nullptr, true, om, ov, &osc);
            });
        }
        G = Gnext;
    }
    if (use_head && !fuse_tail && !tail_early) r.run(slot++, [&] { return launch_tail(tp, c->stream); });
    return r.err;
}

mlp_status hip_fail(mlp_ctx* c, hipError_t e, const char* what) {
    c->poisoned = true;
    c->params_set = 0;
    std::string at;
    if (!c->failed_launch.empty()) at = " (launch " + c->failed_launch + ")";
    c->failed_launch.clear();
    return set_err(c, MLP_ERR_HIP, "%s%s: %s", what, at.c_str(), hipGetErrorString(e));
}

// Writes the guard pattern into every band (creation, and after a band was
// found overwritten).
hipError_t fill_guards(mlp_ctx* c) {
    for (const mlp_ctx::Guard& g : c->guards) {
        const hipError_t e = hipMemsetAsync(c->base + g.off, kGuardByte, g.len, c->stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// With MLP_DEBUG_GUARDS: waits for the stream and compares every guard band
// with its pattern.  A band that changed means a kernel wrote past the end
// of the buffer before it; the call fails with MLP_ERR_GUARD naming that
// buffer, the context is poisoned (the weights may be damaged) and the
// bands are rewritten.  Skipped while the stream is being captured.
mlp_status debug_check(mlp_ctx* c, const char* what) {
    if (!(c->debug & MLP_DEBUG_GUARDS) || capturing(c->stream)) return MLP_OK;
    hipError_t e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, what);
    size_t most = 0;
    for (const mlp_ctx::Guard& g : c->guards) most = std::max(most, g.len);
    std::vector<unsigned char> h(most);
    for (const mlp_ctx::Guard& g : c->guards) {
        e = hipMemcpy(h.data(), c->base + g.off, g.len, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(c, e, what);
        for (size_t i = 0; i < g.len; ++i) {
            if (h[i] == kGuardByte) continue;
            c->poisoned = true;
            c->params_set = 0;
            const unsigned v = h[i];
            e = fill_guards(c);
            if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
            if (e != hipSuccess) return hip_fail(c, e, what);
            return set_err(c, MLP_ERR_GUARD,
                           "%s: guard band after %s overwritten at byte %zu past the buffer's end "
                           "(0x%02x, workspace offset %zu)",
                           what, g.after.c_str(), i, v, g.off + i);
        }
    }
    return MLP_OK;
}

mlp_status check_ready(mlp_ctx* c) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    const unsigned all = c->L >= 32 ? ~0u : ((1u << c->L) - 1u);
    if (c->poisoned && c->params_set != all)
        return set_err(c, MLP_ERR_STATE, "context poisoned by an earlier HIP failure; set every layer");
    if (c->params_set != all)
        return set_err(c, MLP_ERR_STATE, "weights not initialised: call mlp_set_params for every layer");
    return MLP_OK;
}

mlp_status collect_profile(mlp_ctx* c) {
    // Fold completed event pairs into their slots (caller has synchronised).
    std::vector<Pending> keep;
    for (const Pending& p : c->pending) {
        float ms = 0.f;
        const hipError_t e = hipEventElapsedTime(&ms, p.beg, p.end);
        if (e == hipErrorNotReady) {
            keep.push_back(p);
            continue;
        }
        if (e == hipSuccess && p.slot < (int)c->slots[p.kind].size()) {
            c->slots[p.kind][p.slot].total_ms += ms;
            c->slots[p.kind][p.slot].launches += 1;
        }
        c->event_pool.push_back(p.beg);
        c->event_pool.push_back(p.end);
    }
    c->pending.swap(keep);
    return MLP_OK;
}

// ---------------------------------------------------------------- layout --

// Sequential carve of the workspace: every buffer starts on a kAlign
// boundary and is followed by a guard band that runs from its last byte up
// to the next boundary plus kGuardBytes.
struct Layout_ {
    size_t off = 0;
    std::vector<mlp_ctx::Guard> guards;
    size_t take(size_t bytes, std::string name) {
        const size_t o = off;
        const size_t end = align_up(o + bytes, kAlign) + kGuardBytes;
        guards.push_back({std::move(name), o + bytes, end - (o + bytes)});
        off = end;
        return o;
    }
};

mlp_status validate(const mlp_config* cfg, mlp_ctx* tmp) {
    if (!cfg) return set_err(nullptr, MLP_ERR_ARG, "config is NULL");
    if (cfg->n_layers < 1 || cfg->n_layers > kMaxLayers)
        return set_err(nullptr, MLP_ERR_SHAPE, "n_layers %d outside 1..%d", cfg->n_layers, kMaxLayers);
    if (!cfg->dims) return set_err(nullptr, MLP_ERR_ARG, "dims is NULL");
    if (cfg->batch < 1 || cfg->batch > kMaxDim)
        return set_err(nullptr, MLP_ERR_SHAPE, "batch %d outside 1..%d", cfg->batch, kMaxDim);
    if (cfg->precision != MLP_F32 && cfg->precision != MLP_BF16)
        return set_err(nullptr, MLP_ERR_ARG, "unknown precision %d", cfg->precision);
    for (int i = 0; i <= cfg->n_layers; ++i)
        if (cfg->dims[i] < 1 || cfg->dims[i] > kMaxDim)
            return set_err(nullptr, MLP_ERR_SHAPE, "dims[%d] = %d outside 1..%d", i, cfg->dims[i], kMaxDim);
    for (int i = 0; i < cfg->n_layers; ++i)
        if ((int64_t)cfg->dims[i] * cfg->dims[i + 1] > ((int64_t)1 << 31) ||
            (int64_t)cfg->batch * cfg->dims[i] > ((int64_t)1 << 31))
            return set_err(nullptr, MLP_ERR_SHAPE, "layer %d has more than 2^31 elements", i);
    if ((int64_t)cfg->batch * cfg->dims[cfg->n_layers] > ((int64_t)1 << 31))
        return set_err(nullptr, MLP_ERR_SHAPE, "logits have more than 2^31 elements");
    tmp->L = cfg->n_layers;
    for (int i = 0; i <= tmp->L; ++i) tmp->dims[i] = cfg->dims[i];
    tmp->B = cfg->batch;
    tmp->bf16 = cfg->precision == MLP_BF16;
    tmp->stream = (hipStream_t)cfg->stream;
    bool all4 = true;
    for (int i = 0; i <= tmp->L; ++i) all4 = all4 && (tmp->dims[i] % 4 == 0);
    tmp->skinny = !tmp->bf16 && tmp->B <= kSkinnyMaxBatch && all4;
    // Fused output layer: float32, a hidden layer below it, C <= 32, and W_L
    // plus a block of at least 8 activation rows fitting the head's LDS.
    tmp->head = false;
    if (!tmp->bf16 && tmp->L >= 2 && tmp->dims[tmp->L] <= 32) {
        const int H = tmp->dims[tmp->L - 1], C = tmp->dims[tmp->L];
        for (int rb = 64; rb >= 8; rb /= 2)
            if (head_lds_bytes(H, C, rb) <= (size_t)head_max_lds()) {
                tmp->head = true;
                tmp->head_rb = std::min(rb, tmp->B);
                break;
            }
    }
    return MLP_OK;
}

// Plans every product and returns the workspace layout size; with base !=
// nullptr also assigns the buffer pointers.
size_t plan_and_carve(mlp_ctx* c, char* base) {
    const int L = c->L, B = c->B;
    const size_t e = c->bf16 ? 2 : 4;
    size_t max_partial = 0, max_tickets = 1;
    for (int l = 0; l < L; ++l) {
        const int din = c->dims[l], dout = c->dims[l + 1];
        if (c->skinny) {
            c->sfwd[l] = plan_skinny_nn(dout, din, B);
            if (c->sfwd[l].splits > 1) {
                max_partial = std::max(max_partial, (size_t)c->sfwd[l].splits * B * dout);
                max_tickets = std::max(max_tickets, (size_t)c->sfwd[l].tickets);
            }
            {
                // 16 rows of W per workgroup; the columns split too while the
                // row groups alone would leave CUs idle (at least 256 columns
                // per split, a multiple of 32)
                const int rgroups = (din + 15) / 16;
                int cs = std::max(1, std::min((512 + rgroups - 1) / rgroups, dout / 256));
                int kc = (dout + cs - 1) / cs;
                kc = (kc + 31) / 32 * 32;
                cs = (dout + kc - 1) / kc;
                c->sdx[l].splits = cs;
                c->sdx[l].kchunk = kc;
                c->sdx[l].grid = rgroups * cs;
                if (cs > 1 && l > 0) {
                    max_partial = std::max(max_partial, (size_t)cs * B * din);
                    max_tickets = std::max(max_tickets, (size_t)rgroups);
                }
            }
            c->sdw[l].grid = ((dout + 1023) / 1024) * ((din + skinny_tn_rows() - 1) / skinny_tn_rows());
            continue;
        }
        const int vq = c->bf16 ? 8 : 4;
        // 16-byte loads need the layer widths (every leading dimension and
        // contiguous run of the three products) to be multiples of the vector.
        const bool wide = din % vq == 0 && dout % vq == 0;
        // forward NN: A = a_l [B][din] (k-contiguous, K = din), B = W [din][dout]
        c->fwd[l] = plan_gemm(B, dout, din, c->bf16, wide, gemm_big_fits(c->bf16, Layout::NN, B, dout, din, din, dout));
        // dX NT: A = G [B][dout], B = W [din][dout] (both k-contiguous, K = dout)
        c->dx[l] = plan_gemm(B, din, dout, c->bf16, wide, gemm_big_fits(c->bf16, Layout::NT, B, din, dout, dout, dout));
        // dW TN: A = a_l [B][din], B = G [B][dout]: M = din, N = dout, K = B
        c->dw[l] = plan_gemm(din, dout, B, c->bf16, wide, gemm_big_fits(c->bf16, Layout::TN, din, dout, B, din, dout));
        for (const GemmPlan* g : {&c->fwd[l], &c->dx[l], &c->dw[l]})
            if (g->splits > 1) max_tickets = std::max(max_tickets, (size_t)g->tiles_m * g->tiles_n);
        max_partial = std::max(max_partial, partial_elems(c->fwd[l], B, dout));
        max_partial = std::max(max_partial, partial_elems(c->dx[l], B, din));
        max_partial = std::max(max_partial, partial_elems(c->dw[l], din, dout));
    }
    if (c->head && !c->skinny && L >= 2) {
        // the head rides along with the last hidden layer's forward: that
        // launch needs 16 waves and one ticket per 32-row block.  The
        // tickets are reserved whenever the session has the fused output
        // layer, so that mlp_tune may switch that forward to such a plan.
        GemmPlan& g = c->fwd[L - 2];
        if (g.small_waves > 0 && g.cfg == TileCfg::T32x16 &&
            head_lds_bytes(c->dims[L - 1], c->dims[L], 32) <= 64 * 1024)
            g.small_waves = 16;
        max_tickets = std::max(max_tickets, (size_t)(B + 31) / 32);
    }
    int max_hidden = 1;
    for (int l = 1; l < L; ++l) max_hidden = std::max(max_hidden, c->dims[l]);
    const int C = c->dims[L];

    Layout_ lay;
    size_t oW[kMaxLayers], oWb[kMaxLayers], oA[kMaxLayers], oM[kMaxLayers];
    const std::string sl[kMaxLayers + 1] = {"0", "1", "2", "3", "4", "5", "6", "7", "8",
                                            "9", "10", "11", "12", "13", "14", "15", "16"};
    for (int l = 0; l < L; ++l)
        oW[l] = c->external_w ? 0 : lay.take((size_t)c->dims[l] * c->dims[l + 1] * 4, "W" + sl[l]);
    for (int l = 0; l < L; ++l)
        oWb[l] = c->bf16 ? lay.take((size_t)c->dims[l] * c->dims[l + 1] * 2, "W" + sl[l] + " (bf16)") : 0;
    for (int l = 1; l < L; ++l) oA[l] = lay.take((size_t)B * c->dims[l] * e, "a" + sl[l]);
    for (int l = 1; l < L; ++l) oM[l] = lay.take((size_t)B * c->dims[l], "mask" + sl[l]);
    const size_t oXb = c->bf16 ? lay.take((size_t)B * c->dims[0] * 2, "x (bf16)") : 0;
    const size_t oLog = lay.take((size_t)B * C * 4, "logits");
    const size_t oDl = lay.take((size_t)B * C * 4, "dlogits");
    const size_t oDlb = c->bf16 ? lay.take((size_t)B * C * 2, "dlogits (bf16)") : 0;
    const size_t oDz0 = lay.take((size_t)B * max_hidden * e, "dz0");
    const size_t oDz1 = lay.take((size_t)B * max_hidden * e, "dz1");
    c->partial_cap = max_partial;
    c->ticket_cap = max_tickets;
    const size_t oPart = lay.take(max_partial * 4, "split-K partials");
    // counters, the cross-entropy's included, zeroed as whole float4s
    const size_t oTick = lay.take(align_up((max_tickets + 1) * sizeof(unsigned), 16), "counters");
    const size_t oRow = lay.take((size_t)B * 4, "row losses");
    const size_t oLoss = lay.take(16, "loss");
    for (auto& v : c->slots) v.clear();
    if (base) {
        for (int l = 0; l < L; ++l) {
            c->W[l] = c->external_w ? nullptr : (float*)(base + oW[l]);
            c->Wb[l] = c->bf16 ? (bf16_t*)(base + oWb[l]) : nullptr;
        }
        for (int l = 1; l < L; ++l) {
            c->act[l] = base + oA[l];
            c->mask[l] = (uint8_t*)(base + oM[l]);
        }
        c->xb = c->bf16 ? (bf16_t*)(base + oXb) : nullptr;
        c->logits = (float*)(base + oLog);
        c->dlogits = (float*)(base + oDl);
        c->dlogits_b = c->bf16 ? (bf16_t*)(base + oDlb) : nullptr;
        c->dz[0] = base + oDz0;
        c->dz[1] = base + oDz1;
        c->partials = (float*)(base + oPart);
        c->tickets = (unsigned*)(base + oTick);
        c->xent_ticket = c->tickets + max_tickets;
        c->rowloss = (float*)(base + oRow);
        c->loss_slot = (float*)(base + oLoss);
        c->base = base;
        c->guards = std::move(lay.guards);
    }
    return lay.off;
}

size_t tickets_bytes(const mlp_ctx* c) { return align_up((c->ticket_cap + 1) * sizeof(unsigned), 16); }

}  // namespace

// =================================================================== ABI ===

extern "C" {

int32_t mlp_abi_version(void) { return MLP_ABI_VERSION; }

const char* mlp_status_string(mlp_status s) {
    switch (s) {
    case MLP_OK: return "MLP_OK";
    case MLP_ERR_ARG: return "MLP_ERR_ARG";
    case MLP_ERR_SHAPE: return "MLP_ERR_SHAPE";
    case MLP_ERR_WORKSPACE: return "MLP_ERR_WORKSPACE";
    case MLP_ERR_HIP: return "MLP_ERR_HIP";
    case MLP_ERR_STATE: return "MLP_ERR_STATE";
    case MLP_ERR_GUARD: return "MLP_ERR_GUARD";
    }
    return "MLP_ERR_UNKNOWN";
}

const char* mlp_last_error(const mlp_ctx* c) { return c ? c->err.c_str() : g_create_error.c_str(); }

size_t mlp_workspace_bytes(const mlp_config* cfg) {
    mlp_ctx tmp;
    if (validate(cfg, &tmp) != MLP_OK) return 0;
    return plan_and_carve(&tmp, nullptr);
}

mlp_status mlp_create(const mlp_config* cfg, void* workspace, size_t bytes, mlp_ctx** out) {
    g_create_error.clear();
    if (!out) return set_err(nullptr, MLP_ERR_ARG, "out is NULL");
    *out = nullptr;
    mlp_ctx* c = new mlp_ctx();
    mlp_status st = validate(cfg, c);
    if (st != MLP_OK) {
        delete c;
        return st;
    }
    const size_t need = plan_and_carve(c, nullptr);
    if (!workspace || ((uintptr_t)workspace % kAlign) != 0 || bytes < need) {
        delete c;
        return set_err(nullptr, MLP_ERR_WORKSPACE,
                       "workspace %p of %zu bytes: need %zu bytes, %zu-byte aligned", workspace, bytes,
                       need, kAlign);
    }
    plan_and_carve(c, (char*)workspace);
    build_slots(c);
    bool big = false;
    for (int l = 0; l < c->L; ++l)
        for (const GemmPlan* g : {&c->fwd[l], &c->dx[l], &c->dw[l]}) big = big || g->cfg == TileCfg::T256x256;
    if (big) {
        const hipError_t he = gemm_big_prepare();
        if (he != hipSuccess) {
            set_err(nullptr, MLP_ERR_HIP, "large-tile GEMM set-up: %s", hipGetErrorString(he));
            delete c;
            return MLP_ERR_HIP;
        }
    }
    if (c->head) {
        const hipError_t he = head_prepare();
        if (he != hipSuccess) {
            set_err(nullptr, MLP_ERR_HIP, "head kernel set-up: %s", hipGetErrorString(he));
            delete c;
            return MLP_ERR_HIP;
        }
    }
    hipError_t e = hipMemsetAsync(c->tickets, 0, tickets_bytes(c), c->stream);
    if (e == hipSuccess) e = fill_guards(c);
    if (e != hipSuccess) {
        set_err(nullptr, MLP_ERR_HIP, "zeroing counters and filling guard bands: %s", hipGetErrorString(e));
        delete c;
        return MLP_ERR_HIP;
    }
    *out = c;
    return MLP_OK;
}

mlp_status mlp_set_debug(mlp_ctx* c, int32_t flags) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    if (flags & ~(MLP_DEBUG_SYNC | MLP_DEBUG_GUARDS))
        return set_err(c, MLP_ERR_ARG, "unknown debug flags 0x%x", (unsigned)flags);
    c->debug = (unsigned)flags;
    return MLP_OK;
}

void mlp_destroy(mlp_ctx* c) {
    if (!c) return;
    for (const Pending& p : c->pending) {
        hipEventDestroy(p.beg);
        hipEventDestroy(p.end);
    }
    for (hipEvent_t e : c->event_pool) hipEventDestroy(e);
    delete c;
}

mlp_status mlp_set_params(mlp_ctx* c, int32_t layer, const float* w) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    if (layer < 0 || layer >= c->L) return set_err(c, MLP_ERR_ARG, "layer %d outside 0..%d", layer, c->L - 1);
    if (!w || !aligned16(w)) return set_err(c, MLP_ERR_ARG, "w must be a 16-byte aligned device pointer");
    const size_t n = (size_t)c->dims[layer] * c->dims[layer + 1];
    hipError_t e = hipMemcpyAsync(c->W[layer], w, n * 4, hipMemcpyDeviceToDevice, c->stream);
    if (e == hipSuccess && c->bf16) e = launch_cast_bf16(c->W[layer], c->Wb[layer], n, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_set_params");
    c->params_set |= 1u << layer;
    const unsigned all = (1u << c->L) - 1u;
    if (c->params_set == all) c->poisoned = false;
    return MLP_OK;
}

mlp_status mlp_read_params(mlp_ctx* c, int32_t layer, float* dst) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    if (layer < 0 || layer >= c->L) return set_err(c, MLP_ERR_ARG, "layer %d outside 0..%d", layer, c->L - 1);
    if (!dst || !aligned16(dst)) return set_err(c, MLP_ERR_ARG, "dst must be a 16-byte aligned device pointer");
    if (c->poisoned) return set_err(c, MLP_ERR_STATE, "context poisoned by an earlier HIP failure");
    const size_t n = (size_t)c->dims[layer] * c->dims[layer + 1];
    const hipError_t e = hipMemcpyAsync(dst, c->W[layer], n * 4, hipMemcpyDeviceToDevice, c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_read_params");
    return MLP_OK;
}

static mlp_status read_loss(mlp_ctx* c, float* loss) {
    hipError_t e = hipMemcpyAsync(loss, c->loss_slot, 4, hipMemcpyDeviceToHost, c->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "loss read-back");
    if (c->profiling) collect_profile(c);
    return MLP_OK;
}

mlp_status mlp_forward(mlp_ctx* c, const float* x, float* logits, const float* labels, float* loss) {
    mlp_status st = check_ready(c);
    if (st != MLP_OK) return st;
    if (!x || !aligned16(x)) return set_err(c, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (logits && !aligned16(logits)) return set_err(c, MLP_ERR_ARG, "logits must be 16-byte aligned");
    if (labels && !aligned16(labels)) return set_err(c, MLP_ERR_ARG, "labels must be 16-byte aligned");
    hipError_t e = enqueue(c, Mode::Forward, x, labels, 0.f, nullptr, nullptr);
    if (e == hipSuccess && logits)
        e = hipMemcpyAsync(logits, c->logits, (size_t)c->B * c->dims[c->L] * 4, hipMemcpyDeviceToDevice,
                           c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_forward");
    st = debug_check(c, "mlp_forward");
    if (st != MLP_OK) return st;
    if (labels && loss) return read_loss(c, loss);
    return MLP_OK;
}

mlp_status mlp_forward_probs(mlp_ctx* c, const float* x, float* probs) {
    mlp_status st = check_ready(c);
    if (st != MLP_OK) return st;
    if (!x || !aligned16(x)) return set_err(c, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (!probs || !aligned16(probs)) return set_err(c, MLP_ERR_ARG, "probs must be a 16-byte aligned device pointer");
    const hipError_t e = enqueue(c, Mode::Forward, x, nullptr, 0.f, nullptr, nullptr, probs);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_forward_probs");
    return debug_check(c, "mlp_forward_probs");
}

mlp_status mlp_train_step_async(mlp_ctx* c, const float* x, const float* labels, float lr, float* loss_dev) {
    mlp_status st = check_ready(c);
    if (st != MLP_OK) return st;
    if (!x || !aligned16(x)) return set_err(c, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (!labels || !aligned16(labels))
        return set_err(c, MLP_ERR_ARG, "labels must be a 16-byte aligned device pointer");
    if (!std::isfinite(lr)) return set_err(c, MLP_ERR_ARG, "lr must be finite");
    if (loss_dev && ((uintptr_t)loss_dev & 3u)) return set_err(c, MLP_ERR_ARG, "loss_dev must be 4-byte aligned");
    if (c->opt != MLP_OPT_SGD) {
        // the step count is a launch argument of the update: a captured
        // graph would replay one step count forever
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        const hipError_t ce = hipStreamIsCapturing(c->stream, &cs);
        if (ce != hipSuccess) return hip_fail(c, ce, "hipStreamIsCapturing");
        if (cs != hipStreamCaptureStatusNone)
            return set_err(c, MLP_ERR_ARG, "Adam/LaProp steps cannot be captured into a graph (the step count "
                                           "is a launch argument)");
        ++c->opt_t;
    }
    const hipError_t e = enqueue(c, Mode::Train, x, labels, lr, nullptr, loss_dev);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_train_step");
    return debug_check(c, "mlp_train_step");
}

mlp_status mlp_train_steps(mlp_ctx* c, int32_t n, const float* x, const float* labels, float lr,
                           float* loss_dev) {
    mlp_status st = check_ready(c);
    if (st != MLP_OK) return st;
    if (n < 1) return set_err(c, MLP_ERR_ARG, "n must be at least 1");
    if (!x || !aligned16(x)) return set_err(c, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (!labels || !aligned16(labels))
        return set_err(c, MLP_ERR_ARG, "labels must be a 16-byte aligned device pointer");
    if (!std::isfinite(lr)) return set_err(c, MLP_ERR_ARG, "lr must be finite");
    if (loss_dev && ((uintptr_t)loss_dev & 3u)) return set_err(c, MLP_ERR_ARG, "loss_dev must be 4-byte aligned");
    const size_t xs = (size_t)c->B * c->dims[0], ls = (size_t)c->B * c->dims[c->L];
    // every batch of the run must keep the 16-byte alignment of the first
    if (n > 1 && ((xs * 4) % 16 != 0 || (ls * 4) % 16 != 0))
        return set_err(c, MLP_ERR_ARG, "batch rows x width must be a multiple of 4 for a run of steps");
    if (c->opt != MLP_OPT_SGD) {
        // Adam / LaProp: one mlp_train_step_async per batch (its preflight
        // refuses graph capture and advances the step count)
        for (int32_t s = 0; s < n; ++s) {
            st = mlp_train_step_async(c, x + s * xs, labels + s * ls, lr, loss_dev ? loss_dev + s : nullptr);
            if (st != MLP_OK) return st;
        }
        return MLP_OK;
    }
    const bool fuse = steps_fusable(c);
    for (int32_t s = 0; s < n; ++s) {
        const float* xn = (fuse && s + 1 < n) ? x + (s + 1) * xs : nullptr;
        const hipError_t e = enqueue(c, Mode::Train, x + s * xs, labels + s * ls, lr, nullptr,
                                     loss_dev ? loss_dev + s : nullptr, nullptr, fuse && s > 0, xn);
        if (e != hipSuccess) return hip_fail(c, e, "mlp_train_steps");
    }
    return debug_check(c, "mlp_train_steps");
}

}  // extern "C"

// ------------------------------------------------- allocation-free step --
//
// mlp_train_step_static serves callers that cannot allocate device memory:
// every intermediate of the step (activations, masks, logits, dlogits, the
// dZ pair, split-K partials, counters, row losses) lives in `scratch`, a
// static device array of this library (one copy per GPU, held until the
// process ends); the weights stay in the caller's buffers and are updated
// there.  The plan of the last configuration is kept per device and rebuilt
// (host work only) when the configuration changes; the counters are cleared
// with a fill kernel then, and every step leaves them at zero again.
namespace {

constexpr size_t kStaticScratchBytes = MLP_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct StaticPlan {
    char* base = nullptr;     // scratch's device address on this GPU (host code never uses the name)
    mlp_ctx* ctx = nullptr;   // plan of the last configuration run here
    bool zeroed = false;      // counters known to be zero
};

std::mutex g_static_mu;
StaticPlan g_static[kMaxDevices];

bool same_plan_inputs(const mlp_ctx& a, const mlp_ctx& b) {
    if (a.L != b.L || a.B != b.B || a.bf16 != b.bf16 || a.stream != b.stream) return false;
    for (int i = 0; i <= a.L; ++i)
        if (a.dims[i] != b.dims[i]) return false;
    return true;
}

}  // namespace

extern "C" {

mlp_status mlp_train_step_static(const mlp_config* cfg, float* const* weights, const float* x,
                                 const float* labels, float lr, float* loss_dev) {
    g_create_error.clear();
    mlp_ctx probe;
    mlp_status st = validate(cfg, &probe);
    if (st != MLP_OK) return st;
    if (probe.bf16)
        return set_err(nullptr, MLP_ERR_ARG, "the allocation-free step runs float32 sessions only "
                                             "(bf16 sessions keep operand copies of the weights)");
    if (!weights) return set_err(nullptr, MLP_ERR_ARG, "weights is NULL");
    for (int l = 0; l < probe.L; ++l)
        if (!weights[l] || !aligned16(weights[l]))
            return set_err(nullptr, MLP_ERR_ARG, "weights[%d] must be a 16-byte aligned device pointer", l);
    if (!x || !aligned16(x)) return set_err(nullptr, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (!labels || !aligned16(labels))
        return set_err(nullptr, MLP_ERR_ARG, "labels must be a 16-byte aligned device pointer");
    if (!std::isfinite(lr)) return set_err(nullptr, MLP_ERR_ARG, "lr must be finite");
    if (loss_dev && ((uintptr_t)loss_dev & 3u)) return set_err(nullptr, MLP_ERR_ARG, "loss_dev must be 4-byte aligned");
    probe.external_w = true;
    const size_t need = plan_and_carve(&probe, nullptr);
    if (need > kStaticScratchBytes)
        return set_err(nullptr, MLP_ERR_WORKSPACE,
                       "this configuration needs %zu bytes of scratch; the static buffer holds %zu "
                       "(use mlp_create with a workspace)", need, kStaticScratchBytes);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return set_err(nullptr, MLP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return set_err(nullptr, MLP_ERR_ARG, "device %d beyond %d", dev, kMaxDevices);
    if (cfg->stream) {
        // the buffer used is the current device's: the stream must run there
        int sdev = -1;
        e = hipStreamGetDevice((hipStream_t)cfg->stream, &sdev);
        if (e != hipSuccess) return set_err(nullptr, MLP_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return set_err(nullptr, MLP_ERR_ARG, "the stream belongs to device %d but device %d is current", sdev, dev);
    }

    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticPlan& sp = g_static[dev];
    if (!sp.base) {   // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return set_err(nullptr, MLP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        sp.base = (char*)p;
    }
    if (!sp.ctx || !same_plan_inputs(*sp.ctx, probe)) {
        if (!sp.ctx) sp.ctx = new mlp_ctx();
        mlp_ctx* c = sp.ctx;
        *c = mlp_ctx();
        validate(cfg, c);
        c->external_w = true;
        plan_and_carve(c, sp.base);
        build_slots(c);
        sp.zeroed = false;
        if (c->head) {
            e = head_prepare();
            if (e != hipSuccess) {
                delete sp.ctx;
                sp.ctx = nullptr;
                return set_err(nullptr, MLP_ERR_HIP, "head kernel set-up: %s", hipGetErrorString(e));
            }
        }
    }
    mlp_ctx* c = sp.ctx;
    if (!sp.zeroed) {
        // a fill kernel, not a memset, so that the call may be captured
        e = launch_zero((float*)c->tickets, tickets_bytes(c) / sizeof(float), c->stream);
        if (e != hipSuccess) return set_err(nullptr, MLP_ERR_HIP, "clearing counters: %s", hipGetErrorString(e));
        sp.zeroed = true;
    }
    for (int l = 0; l < c->L; ++l) c->W[l] = weights[l];
    c->params_set = c->L >= 32 ? ~0u : ((1u << c->L) - 1u);
    c->poisoned = false;
    e = enqueue(c, Mode::Train, x, labels, lr, nullptr, loss_dev);
    if (e != hipSuccess) {
        sp.zeroed = false;   // a step cut short may leave counters raised
        return set_err(nullptr, MLP_ERR_HIP, "mlp_train_step_static: %s", hipGetErrorString(e));
    }
    return MLP_OK;
}

mlp_status mlp_train_step(mlp_ctx* c, const float* x, const float* labels, float lr, float* loss) {
    mlp_status st = mlp_train_step_async(c, x, labels, lr, nullptr);
    if (st != MLP_OK) return st;
    if (loss) return read_loss(c, loss);
    return MLP_OK;
}

mlp_status mlp_grads(mlp_ctx* c, const float* x, const float* labels, float* const* dw, float* dlogits,
                     float* loss) {
    mlp_status st = check_ready(c);
    if (st != MLP_OK) return st;
    if (!x || !aligned16(x)) return set_err(c, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (!labels || !aligned16(labels))
        return set_err(c, MLP_ERR_ARG, "labels must be a 16-byte aligned device pointer");
    if (!dw) return set_err(c, MLP_ERR_ARG, "dw is NULL");
    for (int l = 0; l < c->L; ++l)
        if (!dw[l] || !aligned16(dw[l])) return set_err(c, MLP_ERR_ARG, "dw[%d] must be a 16-byte aligned device pointer", l);
    if (dlogits && !aligned16(dlogits)) return set_err(c, MLP_ERR_ARG, "dlogits must be 16-byte aligned");
    hipError_t e = enqueue(c, Mode::Grads, x, labels, 0.f, dw, nullptr);
    if (e == hipSuccess && dlogits)
        e = hipMemcpyAsync(dlogits, c->dlogits, (size_t)c->B * c->dims[c->L] * 4, hipMemcpyDeviceToDevice,
                           c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_grads");
    st = debug_check(c, "mlp_grads");
    if (st != MLP_OK) return st;
    if (loss) return read_loss(c, loss);
    return MLP_OK;
}

// Device bytes of an adaptive rule's state: first and second moments,
// float32 per weight, each array 256-byte aligned.
static size_t optimizer_bytes(const mlp_ctx* c) {
    size_t b = 0;
    for (int l = 0; l < c->L; ++l) b += 2 * align_up((size_t)c->dims[l] * c->dims[l + 1] * 4, kAlign);
    return b;
}

size_t mlp_optimizer_bytes(const mlp_config* cfg, int32_t opt) {
    mlp_ctx tmp;
    if (validate(cfg, &tmp) != MLP_OK) return 0;
    if (opt == MLP_OPT_SGD) return 0;
    if (opt != MLP_OPT_ADAM && opt != MLP_OPT_LAPROP) return 0;
    return optimizer_bytes(&tmp);
}

mlp_status mlp_set_optimizer(mlp_ctx* c, int32_t opt, float beta1, float beta2, float eps, void* state,
                             size_t bytes) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    if (opt != MLP_OPT_SGD && opt != MLP_OPT_ADAM && opt != MLP_OPT_LAPROP)
        return set_err(c, MLP_ERR_ARG, "unknown update rule %d", opt);
    if (c->poisoned) return set_err(c, MLP_ERR_STATE, "context poisoned by an earlier HIP failure");
    if (opt != MLP_OPT_SGD) {
        if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
            return set_err(c, MLP_ERR_ARG, "beta1 and beta2 must lie in [0, 1)");
        if (!(eps > 0.f) || !std::isfinite(eps)) return set_err(c, MLP_ERR_ARG, "eps must be finite and > 0");
        const size_t need = optimizer_bytes(c);
        if (!state || ((uintptr_t)state % kAlign) != 0 || bytes < need)
            return set_err(c, MLP_ERR_WORKSPACE, "optimizer state %p of %zu bytes: need %zu bytes, %zu-byte aligned",
                           state, bytes, need, kAlign);
    }
    float* m[kMaxLayers] = {};
    float* v[kMaxLayers] = {};
    if (opt != MLP_OPT_SGD) {
        char* p = (char*)state;
        for (int l = 0; l < c->L; ++l) {
            const size_t a = align_up((size_t)c->dims[l] * c->dims[l + 1] * 4, kAlign);
            m[l] = (float*)p;
            v[l] = (float*)(p + a);
            p += 2 * a;
        }
        // zero both moments (one contiguous range per layer)
        for (int l = 0; l < c->L; ++l) {
            const size_t a = align_up((size_t)c->dims[l] * c->dims[l + 1] * 4, kAlign);
            const hipError_t e = launch_zero(m[l], 2 * a / 4, c->stream);
            if (e != hipSuccess) return hip_fail(c, e, "zeroing the moments");
        }
    }
    c->opt = opt;
    c->opt_b1 = beta1;
    c->opt_b2 = beta2;
    c->opt_eps = eps;
    c->opt_t = 0;
    for (int l = 0; l < kMaxLayers; ++l) {
        c->opt_m[l] = m[l];
        c->opt_v[l] = v[l];
    }
    // the launch sequence of a step changed: new slot names, fresh counts
    collect_profile(c);
    for (const Pending& pe : c->pending) {
        hipEventDestroy(pe.beg);
        hipEventDestroy(pe.end);
    }
    c->pending.clear();
    build_slots(c);
    return MLP_OK;
}

// ------------------------------------------------------------ checkpoints --
// Layout (little-endian, host memory): a 136-byte header, then the payload:
// every W_l as float32 [dims[l]][dims[l+1]] row-major without padding, then,
// when the checkpoint carries an adaptive rule's state, every m_l and then
// every v_l in the same shapes.  The header's checksum (ckpt_hash) runs the
// FNV-1a step over the payload's 64-bit words in four interleaved lanes.
namespace {

constexpr char kCkptMagic[8] = {'M', 'L', 'P', 'C', 'K', 'P', 'T', '1'};
constexpr uint32_t kCkptVersion = 2;

struct CkptHeader {
    char magic[8];
    uint32_t version;
    uint32_t n_layers;
    uint32_t precision;      // of the session that wrote it (informational)
    uint32_t optimizer;      // MLP_OPT_*; 0 = no moments in the payload
    int32_t dims[kMaxLayers + 1];
    float beta1, beta2, eps;
    uint32_t reserved[2];    // zero
    int64_t step;            // steps taken with the moments
    uint64_t payload_bytes;
    uint64_t checksum;
};
static_assert(sizeof(CkptHeader) == 136, "checkpoint header layout: no implicit padding");

// FNV-1a, 64-bit (Fowler, Noll and Vo): offset basis 0xcbf29ce484222325,
// prime 0x100000001b3.
constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

// Payload checksum: the bytes read as little-endian 64-bit words (a last
// 4-byte remainder zero-extended); word i goes to lane i mod 4, each lane
// starting at the FNV-1a basis and taking h = (h ^ word) * prime; the result
// is byte-wise FNV-1a over the four lanes' 32 little-endian bytes, lane 0
// first.  Four independent multiply chains: several GB/s on one host core,
// where byte-wise FNV-1a over the whole payload ran near 1 GB/s.
uint64_t ckpt_hash(const unsigned char* p, size_t n) {
    uint64_t h[4] = {kFnvBasis, kFnvBasis, kFnvBasis, kFnvBasis};
    const size_t nw = n / 8;
    size_t i = 0;
    for (; i + 4 <= nw; i += 4) {
        uint64_t w[4];
        std::memcpy(w, p + 8 * i, 32);
        for (int l = 0; l < 4; ++l) h[l] = (h[l] ^ w[l]) * kFnvPrime;
    }
    for (; i < nw; ++i) {
        uint64_t w;
        std::memcpy(&w, p + 8 * i, 8);
        h[i % 4] = (h[i % 4] ^ w) * kFnvPrime;
    }
    if (n % 8) {
        uint64_t w = 0;
        std::memcpy(&w, p + 8 * nw, n % 8);
        h[nw % 4] = (h[nw % 4] ^ w) * kFnvPrime;
    }
    uint64_t r = kFnvBasis;
    for (int l = 0; l < 4; ++l)
        for (int b = 0; b < 8; ++b) {
            r ^= (h[l] >> (8 * b)) & 0xffu;
            r *= kFnvPrime;
        }
    return r;
}

size_t ckpt_payload(int L, const int32_t* dims, bool moments) {
    size_t n = 0;
    for (int l = 0; l < L; ++l) n += (size_t)dims[l] * dims[l + 1];
    return n * 4 * (moments ? 3 : 1);
}

// Header and payload checks shared by mlp_checkpoint_info and the load
// preflight; no device memory is touched.
mlp_status ckpt_check(const void* src, size_t bytes, CkptHeader* h, std::string* why) {
    char buf[160];
    if (!src) {
        *why = "checkpoint pointer is NULL";
        return MLP_ERR_ARG;
    }
    if (bytes < sizeof(CkptHeader)) {
        std::snprintf(buf, sizeof buf, "checkpoint of %zu bytes is shorter than its %zu-byte header", bytes,
                      sizeof(CkptHeader));
        *why = buf;
        return MLP_ERR_ARG;
    }
    std::memcpy(h, src, sizeof(CkptHeader));
    if (std::memcmp(h->magic, kCkptMagic, 8) != 0) {
        *why = "not a checkpoint (magic)";
        return MLP_ERR_ARG;
    }
    if (h->version != kCkptVersion) {
        std::snprintf(buf, sizeof buf, "checkpoint version %u, this library reads %u", h->version, kCkptVersion);
        *why = buf;
        return MLP_ERR_ARG;
    }
    if (h->n_layers < 1 || h->n_layers > (uint32_t)kMaxLayers || h->optimizer > MLP_OPT_LAPROP) {
        *why = "checkpoint header out of range (layers or update rule)";
        return MLP_ERR_ARG;
    }
    for (uint32_t i = 0; i <= h->n_layers; ++i)
        if (h->dims[i] < 1 || h->dims[i] > kMaxDim) {
            *why = "checkpoint header out of range (dims)";
            return MLP_ERR_ARG;
        }
    const size_t want = ckpt_payload((int)h->n_layers, h->dims, h->optimizer != MLP_OPT_SGD);
    if (h->payload_bytes != want || bytes < sizeof(CkptHeader) + want) {
        std::snprintf(buf, sizeof buf, "checkpoint payload: header says %llu bytes, shapes need %zu, buffer holds %zu",
                      (unsigned long long)h->payload_bytes, want, bytes - sizeof(CkptHeader));
        *why = buf;
        return MLP_ERR_ARG;
    }
    if (ckpt_hash((const unsigned char*)src + sizeof(CkptHeader), want) != h->checksum) {
        *why = "checkpoint checksum mismatch (payload damaged)";
        return MLP_ERR_ARG;
    }
    return MLP_OK;
}

}  // namespace

size_t mlp_checkpoint_bytes(const mlp_ctx* c, int32_t with_optimizer) {
    if (!c) return 0;
    const bool mom = with_optimizer && c->opt != MLP_OPT_SGD;
    return sizeof(CkptHeader) + ckpt_payload(c->L, c->dims, mom);
}

mlp_status mlp_save_checkpoint(mlp_ctx* c, void* dst, size_t bytes, int32_t with_optimizer) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    if (c->poisoned) return set_err(c, MLP_ERR_STATE, "context poisoned by an earlier HIP failure");
    const unsigned all = (1u << c->L) - 1u;
    if (c->params_set != all) return set_err(c, MLP_ERR_STATE, "weights not initialised: nothing to save");
    const bool mom = with_optimizer && c->opt != MLP_OPT_SGD;
    const size_t need = mlp_checkpoint_bytes(c, with_optimizer);
    if (!dst || bytes < need) return set_err(c, MLP_ERR_ARG, "checkpoint buffer %p of %zu bytes: need %zu", dst, bytes, need);
    CkptHeader h{};
    std::memcpy(h.magic, kCkptMagic, 8);
    h.version = kCkptVersion;
    h.n_layers = (uint32_t)c->L;
    h.precision = c->bf16 ? MLP_BF16 : MLP_F32;
    h.optimizer = mom ? (uint32_t)c->opt : 0u;
    for (int i = 0; i <= c->L; ++i) h.dims[i] = c->dims[i];
    h.beta1 = mom ? c->opt_b1 : 0.f;
    h.beta2 = mom ? c->opt_b2 : 0.f;
    h.eps = mom ? c->opt_eps : 0.f;
    h.step = mom ? c->opt_t : 0;
    h.payload_bytes = ckpt_payload(c->L, c->dims, mom);
    unsigned char* out = (unsigned char*)dst + sizeof(CkptHeader);
    // pending work on the stream (the last step) must finish first
    hipError_t e = hipStreamSynchronize(c->stream);
    size_t off = 0;
    for (int part = 0; part < (mom ? 3 : 1) && e == hipSuccess; ++part)
        for (int l = 0; l < c->L && e == hipSuccess; ++l) {
            const size_t n = (size_t)c->dims[l] * c->dims[l + 1] * 4;
            const float* srcp = part == 0 ? c->W[l] : (part == 1 ? c->opt_m[l] : c->opt_v[l]);
            e = hipMemcpy(out + off, srcp, n, hipMemcpyDeviceToHost);
            off += n;
        }
    if (e != hipSuccess) return hip_fail(c, e, "mlp_save_checkpoint");
    h.checksum = ckpt_hash(out, h.payload_bytes);
    std::memcpy(dst, &h, sizeof h);
    return MLP_OK;
}

mlp_status mlp_checkpoint_info(const void* src, size_t bytes, int32_t* n_layers, int32_t* dims,
                               int32_t* optimizer, int64_t* step) {
    CkptHeader h;
    std::string why;
    g_create_error.clear();
    const mlp_status st = ckpt_check(src, bytes, &h, &why);
    if (st != MLP_OK) return set_err(nullptr, st, "%s", why.c_str());
    if (n_layers) *n_layers = (int32_t)h.n_layers;
    if (dims)
        for (uint32_t i = 0; i <= h.n_layers; ++i) dims[i] = h.dims[i];
    if (optimizer) *optimizer = (int32_t)h.optimizer;
    if (step) *step = h.step;
    return MLP_OK;
}

mlp_status mlp_load_checkpoint(mlp_ctx* c, const void* src, size_t bytes) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    // preflight: everything is checked before any device memory changes
    CkptHeader h;
    std::string why;
    mlp_status st = ckpt_check(src, bytes, &h, &why);
    if (st != MLP_OK) return set_err(c, st, "%s", why.c_str());
    if ((int)h.n_layers != c->L) return set_err(c, MLP_ERR_SHAPE, "checkpoint has %u layers, the session %d", h.n_layers, c->L);
    for (int i = 0; i <= c->L; ++i)
        if (h.dims[i] != c->dims[i])
            return set_err(c, MLP_ERR_SHAPE, "checkpoint width d%d = %d, the session has %d", i, h.dims[i], c->dims[i]);
    if (c->opt != MLP_OPT_SGD) {
        if (h.optimizer != (uint32_t)c->opt)
            return set_err(c, MLP_ERR_ARG, "the session uses update rule %d but the checkpoint carries %s", c->opt,
                           h.optimizer ? "another rule's state" : "no optimizer state");
        if (h.beta1 != c->opt_b1 || h.beta2 != c->opt_b2 || h.eps != c->opt_eps)
            return set_err(c, MLP_ERR_ARG, "checkpoint betas/eps differ from the session's");
    }
    const unsigned char* in = (const unsigned char*)src + sizeof(CkptHeader);
    const bool mom = c->opt != MLP_OPT_SGD;   // moments restored only into a session using them
    hipError_t e = hipSuccess;
    size_t off = 0;
    for (int part = 0; part < (h.optimizer != MLP_OPT_SGD ? 3 : 1) && e == hipSuccess; ++part)
        for (int l = 0; l < c->L && e == hipSuccess; ++l) {
            const size_t n = (size_t)c->dims[l] * c->dims[l + 1] * 4;
            float* dstp = part == 0 ? c->W[l] : (part == 1 ? c->opt_m[l] : c->opt_v[l]);
            if (part == 0 || mom) e = hipMemcpyAsync(dstp, in + off, n, hipMemcpyHostToDevice, c->stream);
            off += n;
        }
    for (int l = 0; l < c->L && e == hipSuccess && c->bf16; ++l)
        e = launch_cast_bf16(c->W[l], c->Wb[l], (size_t)c->dims[l] * c->dims[l + 1], c->stream);
    // the source is caller memory that may be reused at once
    if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_load_checkpoint");
    if (mom) c->opt_t = h.step;
    c->params_set = (1u << c->L) - 1u;
    c->poisoned = false;
    return MLP_OK;
}

// ---------------------------------------------------------------- tuning --
// A bounded search over launch plans (the README's MEGANEURA_TUNE /
// tune_with): for each product, the large-tile bf16 kernel with K split 1, 2
// or 4, the tiled kernels' 128x128 / 128x64 / 64x64 tiles with K split 1..8,
// and for the under-filled f32 products the small-product kernel's 4, 8 or
// 16 waves on 32x16 or 32x32 tiles -- every candidate within the buffers the
// context planned at creation.  Plans that the fused output layer relies on
// are kept.
namespace {

std::vector<GemmPlan> gemm_candidates(const mlp_ctx* c, int M, int N, int K, bool kvec_ok, bool big_ok,
                                      const GemmPlan& cur) {
    std::vector<GemmPlan> out;
    auto fits = [&](const GemmPlan& g) {
        if (partial_elems(g, M, N) > c->partial_cap) return false;
        if (g.splits > 1 && g.cfg != TileCfg::T256x256 && g.small_waves == 0 &&
            (size_t)g.tiles_m * g.tiles_n > c->ticket_cap)
            return false;
        return true;
    };
    auto same = [](const GemmPlan& a, const GemmPlan& b) {
        return a.cfg == b.cfg && a.splits == b.splits && a.small_waves == b.small_waves && a.kchunk == b.kchunk;
    };
    auto push = [&](const GemmPlan& g) {
        if (!fits(g)) return;
        for (const GemmPlan& o : out)
            if (same(o, g)) return;
        out.push_back(g);
    };
    push(cur);
    auto split = [&](GemmPlan g, int s, int bk) {
        int kchunk = (K + s - 1) / s;
        kchunk = (kchunk + bk - 1) / bk * bk;
        s = (K + kchunk - 1) / kchunk;
        g.splits = s;
        g.kchunk = s > 1 ? kchunk : std::max(K, 1);
        g.grid = g.tiles_m * g.tiles_n * s;
        return g;
    };
    if (big_ok) {
        for (int s : {1, 2, 4}) {
            GemmPlan g;
            g.cfg = TileCfg::T256x256;
            g.tiles_m = (M + 255) / 256;
            g.tiles_n = (N + 255) / 256;
            g.vec = c->bf16 ? 8 : 4;
            if (s > 1 && K / s < 512) continue;
            push(split(g, s, c->bf16 ? 64 : 32));
        }
    }
    const int bk = c->bf16 ? 64 : 32, kmin = c->bf16 ? 256 : 128;
    for (TileCfg cfg : {TileCfg::T128x128, TileCfg::T128x64, TileCfg::T64x64}) {
        int bm, bn;
        tile_shape(cfg, &bm, &bn);
        for (int s : {1, 2, 4, 8}) {
            if (s > 1 && K / s < kmin) continue;
            GemmPlan g;
            g.cfg = cfg;
            g.tiles_m = (M + bm - 1) / bm;
            g.tiles_n = (N + bn - 1) / bn;
            g.vec = kvec_ok ? (c->bf16 ? 8 : 4) : 1;
            push(split(g, s, bk));
        }
    }
    if (!c->bf16 && cur.small_waves > 0) {
        for (int nw : {4, 8, 16})
            for (TileCfg cfg : {TileCfg::T32x16, TileCfg::T32x32}) {
                GemmPlan g;
                g.cfg = cfg;
                g.small_waves = nw;
                g.splits = 1;
                g.kchunk = std::max(K, 1);
                g.tiles_m = (M + 31) / 32;
                g.tiles_n = cfg == TileCfg::T32x16 ? (N + 15) / 16 : (N + 31) / 32;
                g.grid = g.tiles_m * g.tiles_n;
                g.vec = kvec_ok ? 4 : 1;
                push(g);
            }
    }
    return out;
}

}  // namespace

mlp_status mlp_tune(mlp_ctx* c, const float* x, const float* labels, int32_t repeats) {
    mlp_status st = check_ready(c);
    if (st != MLP_OK) return st;
    if (!x || !aligned16(x)) return set_err(c, MLP_ERR_ARG, "x must be a 16-byte aligned device pointer");
    if (!labels || !aligned16(labels))
        return set_err(c, MLP_ERR_ARG, "labels must be a 16-byte aligned device pointer");
    if (repeats < 1 || repeats > 100) return set_err(c, MLP_ERR_ARG, "repeats must lie in 1..100");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(c->stream, &cs);
    if (e != hipSuccess) return hip_fail(c, e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone) return set_err(c, MLP_ERR_ARG, "tuning cannot run under stream capture");
    // Timed steps are SGD steps with lr = 0: W - 0 * dW leaves every finite
    // weight as it is and no optimizer state is touched.
    const int opt = c->opt;
    const bool prof = c->profiling;
    c->opt = MLP_OPT_SGD;
    e = hipStreamSynchronize(c->stream);
    if (e != hipSuccess) return hip_fail(c, e, "mlp_tune");
    collect_profile(c);
    auto step_ms = [&](double* ms) -> hipError_t {
        c->profiling = false;
        hipError_t he = enqueue(c, Mode::Train, x, labels, 0.f, nullptr, nullptr);   // warm-up
        c->profiling = true;
        for (auto& v : c->slots)
            for (Slot& sl : v) sl.total_ms = 0, sl.launches = 0;
        for (int i = 0; i < repeats && he == hipSuccess; ++i)
            he = enqueue(c, Mode::Train, x, labels, 0.f, nullptr, nullptr);
        if (he == hipSuccess) he = hipStreamSynchronize(c->stream);
        collect_profile(c);
        double t = 0;
        for (const Slot& sl : c->slots[kStep]) t += sl.total_ms;
        *ms = t / repeats;
        return he;
    };
    const int L = c->L, B = c->B;
    // Keep a candidate only on a clear win (2%) over the best so far.
    auto choose = [&](auto* plan, const auto& cands) {
        auto best = *plan;
        double best_ms = 0;
        e = step_ms(&best_ms);
        for (size_t i = 0; i < cands.size() && e == hipSuccess; ++i) {
            *plan = cands[i];
            double ms = 0;
            e = step_ms(&ms);
            if (e == hipSuccess && ms < 0.98 * best_ms) {
                best = cands[i];
                best_ms = ms;
            }
        }
        *plan = best;
    };
    if (c->skinny) {
        // Skinny sessions: the K splits of each forward pass and the column
        // splits of each fused dX + dW pass, within the planned workspace.
        for (int l = 0; l < L && e == hipSuccess; ++l) {
            const int din = c->dims[l], dout = c->dims[l + 1];
            std::vector<SkinnyPlan> fc;
            const int ncg = (dout + 63) / 64;
            for (int want : {1, 2, 4, 8, 16, 32}) {
                SkinnyPlan s = c->sfwd[l];
                int kchunk = (din + want - 1) / want;
                kchunk = (kchunk + 15) / 16 * 16;
                const int sp = (din + kchunk - 1) / kchunk;
                if (sp == c->sfwd[l].splits) continue;
                if (sp > 1 && ((size_t)sp * B * dout > c->partial_cap || (size_t)ncg > c->ticket_cap)) continue;
                s.splits = sp;
                s.kchunk = sp > 1 ? kchunk : din;
                s.grid = ncg * sp;
                s.tickets = ncg;
                fc.push_back(s);
            }
            choose(&c->sfwd[l], fc);
            if (l == 0 || e != hipSuccess) continue;
            std::vector<SkinnyPlan> xc;
            const int rgroups = (din + 15) / 16;
            for (int want : {1, 2, 4, 8, 16}) {
                SkinnyPlan s = c->sdx[l];
                int kc = (dout + want - 1) / want;
                kc = (kc + 31) / 32 * 32;
                const int cs = (dout + kc - 1) / kc;
                if (cs == c->sdx[l].splits) continue;
                if (cs > 1 && ((size_t)cs * B * din > c->partial_cap || (size_t)rgroups > c->ticket_cap)) continue;
                s.splits = cs;
                s.kchunk = kc;
                s.grid = rgroups * cs;
                xc.push_back(s);
            }
            choose(&c->sdx[l], xc);
        }
    }
    for (int l = 0; l < L && e == hipSuccess && !c->skinny; ++l) {
        const int din = c->dims[l], dout = c->dims[l + 1];
        const int vq = c->bf16 ? 8 : 4;
        const bool wide = din % vq == 0 && dout % vq == 0;
        struct Item {
            GemmPlan* g;
            int M, N, K;
            bool big;
            bool used;
        } items[3] = {
            {&c->fwd[l], B, dout, din, gemm_big_fits(c->bf16, Layout::NN, B, dout, din, din, dout),
             !(c->head && l == L - 1) && !(head_fused(c) && l == L - 2)},
            {&c->dx[l], B, din, dout, gemm_big_fits(c->bf16, Layout::NT, B, din, dout, dout, dout),
             l > 0 && !(c->head && l == L - 1)},
            {&c->dw[l], din, dout, B, gemm_big_fits(c->bf16, Layout::TN, din, dout, B, din, dout),
             !(c->head && l == L - 1) && !(tail_fused(c) && l == 0)},
        };
        for (Item& it : items) {
            if (!it.used || e != hipSuccess) continue;
            const std::vector<GemmPlan> cands = gemm_candidates(c, it.M, it.N, it.K, wide, it.big, *it.g);
            if (cands.size() < 2) continue;
            GemmPlan best = *it.g;
            double best_ms = 0;
            e = step_ms(&best_ms);
            for (size_t i = 1; i < cands.size() && e == hipSuccess; ++i) {
                *it.g = cands[i];
                double ms = 0;
                e = step_ms(&ms);
                if (e == hipSuccess && ms < 0.98 * best_ms) {   // a clear win only
                    best = cands[i];
                    best_ms = ms;
                }
            }
            *it.g = best;
        }
    }
    c->opt = opt;
    c->profiling = prof;
    if (e != hipSuccess) return hip_fail(c, e, "mlp_tune");
    build_slots(c);   // plan changes can change which launches are fused
    return debug_check(c, "mlp_tune");
}

mlp_status mlp_read_state(mlp_ctx* c, int32_t which, int32_t layer, void* dst) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    if (!dst || !aligned16(dst)) return set_err(c, MLP_ERR_ARG, "dst must be a 16-byte aligned device pointer");
    if (c->poisoned) return set_err(c, MLP_ERR_STATE, "context poisoned by an earlier HIP failure");
    const size_t BC = (size_t)c->B * c->dims[c->L];
    hipError_t e = hipSuccess;
    switch (which) {
    case MLP_STATE_ACT:
    case MLP_STATE_MASK: {
        if (layer < 1 || layer >= c->L)
            return set_err(c, MLP_ERR_ARG, "layer %d outside 1..%d", layer, c->L - 1);
        const size_t n = (size_t)c->B * c->dims[layer];
        if (which == MLP_STATE_MASK)
            e = hipMemcpyAsync(dst, c->mask[layer], n, hipMemcpyDeviceToDevice, c->stream);
        else if (c->bf16)
            e = launch_widen_bf16((const bf16_t*)c->act[layer], (float*)dst, n, c->stream);
        else
            e = hipMemcpyAsync(dst, c->act[layer], n * 4, hipMemcpyDeviceToDevice, c->stream);
        break;
    }
    case MLP_STATE_DLOGITS:
        e = hipMemcpyAsync(dst, c->dlogits, BC * 4, hipMemcpyDeviceToDevice, c->stream);
        break;
    case MLP_STATE_LOGITS:
        e = hipMemcpyAsync(dst, c->logits, BC * 4, hipMemcpyDeviceToDevice, c->stream);
        break;
    default:
        return set_err(c, MLP_ERR_ARG, "unknown state kind %d", which);
    }
    if (e != hipSuccess) return hip_fail(c, e, "mlp_read_state");
    return MLP_OK;
}

mlp_status mlp_profile_enable(mlp_ctx* c, int32_t enable) {
    if (!c) return MLP_ERR_ARG;
    c->profiling = enable != 0;
    return MLP_OK;
}

mlp_status mlp_profile_reset(mlp_ctx* c) {
    if (!c) return MLP_ERR_ARG;
    collect_profile(c);
    for (auto& v : c->slots)
        for (Slot& s : v) {
            s.total_ms = 0;
            s.launches = 0;
        }
    return MLP_OK;
}

int32_t mlp_profile_slots(const mlp_ctx* c) { return c ? (int32_t)c->slots[c->prof_kind].size() : 0; }

mlp_status mlp_profile_read(mlp_ctx* c, int32_t idx, char* name, size_t name_len, double* total_ms,
                            int64_t* launches, double* flops, double* bytes) {
    if (!c) return MLP_ERR_ARG;
    c->err.clear();
    const std::vector<Slot>& slots = c->slots[c->prof_kind];
    if (idx < 0 || idx >= (int32_t)slots.size()) return set_err(c, MLP_ERR_ARG, "slot %d out of range", idx);
    collect_profile(c);
    const Slot& s = slots[idx];
    if (name && name_len) {
        std::strncpy(name, s.name.c_str(), name_len - 1);
        name[name_len - 1] = 0;
    }
    if (total_ms) *total_ms = s.total_ms;
    if (launches) *launches = s.launches;
    if (flops) *flops = s.flops;
    if (bytes) *bytes = s.bytes;
    return MLP_OK;
}

}  // extern "C"
