/*
 * mlp.h -- C ABI of libmlp.so: the compiled training step of a bias-free ReLU
 * MLP on one AMD Instinct MI355X (gfx950).
 *
 * The graph is the one in the Meganeura README ("Example" section):
 *     h      = relu(matmul(x, w1))          ... repeated for every hidden layer
 *     logits = matmul(h, wL)
 *     loss   = cross_entropy_loss(logits, labels)
 * with the backward pass the framework's autodiff derives for it and a plain
 * SGD update (README "Contents": SGD sessions), or Adam / LaProp with moments
 * kept only when requested (mlp_set_optimizer).  A step is a fixed sequence
 * of hand-written HIP kernels: MFMA GEMMs with fused ReLU/mask, mask-multiply
 * and SGD epilogues, and one row-wise softmax cross-entropy kernel.  For
 * narrow outputs (float32, at most 32 classes) the last layer's products,
 * the cross-entropy and the loss mean run inside the neighbouring GEMM
 * launches, and for batches of at most 16 rows every product is one
 * streaming pass over its weight matrix.  mlp_train_step_async enqueues
 * kernels only (no memsets, no host synchronisation), so it may be captured
 * into a HIP graph.
 *
 * Two arithmetic contracts, following the split between a strict-f32 mode
 * and validated fast paths in the abstract of "Meganeura: Portable GPU
 * Training and Inference through Vulkan and Metal":
 *   MLP_F32  -- every product and sum in IEEE float32 (f32 MFMA);
 *   MLP_BF16 -- GEMM operands rounded to bfloat16 (round-to-nearest-even),
 *               float32 accumulation, float32 softmax-CE, float32 master
 *               weights and update.
 *
 * Conventions for every entry point
 *   - Layers are numbered 0 .. n_layers-1; weight l has shape
 *     [dims[l], dims[l+1]] ([in, out], out = in @ W, as in the README).
 *   - Every tensor is row-major and contiguous with its logical shape; no
 *     padding is visible (README "Contents" says checkpoints keep tensors at
 *     their logical shapes, free of the device's padding).
 *   - Pointers named *dev* or documented as device pointers are HIP device
 *     memory, 16-byte aligned; they are owned by the caller.  Host pointers
 *     are documented as such.
 *   - The library never allocates device memory: all of its state lives in
 *     the caller-provided workspace, which must stay alive until
 *     mlp_destroy.  All device work is enqueued on the config's stream, and
 *     inputs must be ready in that stream's order.  One context may be used
 *     by one host thread at a time; calls on one context are not
 *     re-entrant.
 *   - Values are not checked.  A NaN in x, the labels or the weights
 *     propagates: the ReLU keeps a NaN pre-activation (as the definition
 *     a = z * [z > 0] does), so it reaches the logits and the loss, and the
 *     call returns MLP_OK; weights updated by such a step are not meaningful
 *     (README "Debugging" leaves reports of NaN outputs to a separate scan).
 *   - Every argument is checked before anything is enqueued (README
 *     "Contents": a restore is validated in full before it changes any
 *     state; the same rule applies to every call here): on an error return the
 *     context and device state are unchanged, and mlp_last_error() describes
 *     the problem.  A HIP failure after work was enqueued returns
 *     MLP_ERR_HIP and poisons the context: later calls return MLP_ERR_STATE
 *     until mlp_set_params has been called for every layer.
 */
#ifndef MLP_H_
#define MLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLP_ABI_VERSION 1

typedef struct mlp_ctx mlp_ctx;

typedef enum mlp_status {
    MLP_OK = 0,
    MLP_ERR_ARG = 1,        /* null/misaligned pointer, bad index, non-finite lr */
    MLP_ERR_SHAPE = 2,      /* dims or batch outside the supported range */
    MLP_ERR_WORKSPACE = 3,  /* workspace null, too small or misaligned */
    MLP_ERR_HIP = 4,        /* a HIP runtime call failed */
    MLP_ERR_STATE = 5,      /* context poisoned by an earlier HIP failure */
    MLP_ERR_GUARD = 6       /* a guard band of the workspace was overwritten (MLP_DEBUG_GUARDS) */
} mlp_status;

typedef enum mlp_precision {
    MLP_F32 = 0,
    MLP_BF16 = 1
} mlp_precision;

/* Update rule of a training step (README "Contents": Adam/LaProp moments are
 * allocated only when requested; SGD sessions keep no optimizer state). */
typedef enum mlp_optimizer {
    MLP_OPT_SGD = 0,        /* W <- W - lr g */
    MLP_OPT_ADAM = 1,       /* Kingma and Ba, "Adam: A Method for Stochastic Optimization",
                               Algorithm 1: m <- b1 m + (1-b1) g, v <- b2 v + (1-b2) g^2,
                               W <- W - lr (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps) */
    MLP_OPT_LAPROP = 2      /* Ziyin, Wang and Ueda, "LaProp: Separating Momentum and
                               Adaptivity in Adam", Algorithm 1: v <- b2 v + (1-b2) g^2,
                               m <- b1 m + (1-b1) g / (sqrt(v/(1-b2^t)) + eps),
                               W <- W - lr m/(1-b1^t) */
} mlp_optimizer;

/* What mlp_read_state copies out (debug-session reads, README "Debugging"). */
typedef enum mlp_state_kind {
    MLP_STATE_ACT = 0,      /* a_l = relu(z_l), l = 1..n_layers-1: float32 [B, dims[l]]
                               (bf16 activations are widened to float32) */
    MLP_STATE_MASK = 1,     /* m_l = [z_l > 0], l = 1..n_layers-1: uint8 [B, dims[l]] */
    MLP_STATE_DLOGITS = 2,  /* dloss/dlogits of the last step: float32 [B, C] (layer ignored) */
    MLP_STATE_LOGITS = 3    /* logits of the last forward: float32 [B, C] (layer ignored) */
} mlp_state_kind;

/* Static shape of the graph: fixed at creation, as the README's typed
 * static graph fixes input shapes (g.input("x", &[32, 784])). */
typedef struct mlp_config {
    int32_t n_layers;        /* number of weight matrices L, 1 <= L <= 16 */
    const int32_t* dims;     /* host array of L+1 widths d0..dL, each 1 .. 1<<20 */
    int32_t batch;           /* B, 1 .. 1<<20 */
    int32_t precision;       /* mlp_precision */
    void* stream;            /* hipStream_t for all work; NULL = the null stream */
} mlp_config;

/* Library ABI version (MLP_ABI_VERSION). */
int32_t mlp_abi_version(void);

/* Device workspace the configuration needs, in bytes (a multiple of 256);
 * 0 if the configuration is invalid.  Host only.  The session's buffer plan
 * (README "Environment variables": buffers are planned at build with
 * lifetime aliasing, MEGANEURA_NO_ALIAS / MEGANEURA_DUMP_PLAN) made static:
 * weights, activations, masks, a ping-pong pair of gradient buffers, split-K
 * partials and counters, laid out once for this shape.  Each buffer starts
 * on a 256-byte boundary and is followed by a guard band of at least 256
 * bytes (see mlp_set_debug). */
size_t mlp_workspace_bytes(const mlp_config* cfg);

/* Create a context that lives in `workspace` (device memory of at least
 * mlp_workspace_bytes(cfg) bytes, 256-byte aligned, owned by the caller).
 * Enqueues the zeroing of the library's counters and the filling of the
 * guard bands (hipMemsetAsync) on cfg->stream.  The
 * weights are undefined until mlp_set_params has been called for every
 * layer.  The analogue of the README's build_session: kernels are compiled
 * ahead of time, so this only plans buffers and launch shapes. */
mlp_status mlp_create(const mlp_config* cfg, void* workspace, size_t bytes, mlp_ctx** out);

/* Free the host-side context (the end of the session that README "Example"
 * builds with build_session).  Device memory is the caller's; NULL is
 * ignored. */
void mlp_destroy(mlp_ctx* ctx);

/* Copy weight `layer` in: w is a device float32 [dims[layer], dims[layer+1]]
 * array (the parameter g.parameter("w1", &[784, 128]) of README "Example";
 * the upload the README's "Environment variables" table calls
 * set_parameter).  In MLP_BF16 mode the bfloat16 operand copy is refreshed
 * too.  Errors: MLP_ERR_ARG (layer out of range, w NULL or not 16-byte
 * aligned), MLP_ERR_HIP. */
mlp_status mlp_set_params(mlp_ctx* ctx, int32_t layer, const float* w);

/* Copy the float32 master of weight `layer` out to device memory `dst`
 * ([dims[layer], dims[layer+1]]), in stream order: the analogue of
 * read_node_by_name on a parameter (README "Debugging": debug sessions read
 * materialised values after a step).  Errors: MLP_ERR_ARG, MLP_ERR_STATE
 * (context poisoned), MLP_ERR_HIP. */
mlp_status mlp_read_params(mlp_ctx* ctx, int32_t layer, float* dst);

/* Forward pass only: the graph of README "Example" up to its logits (and
 * the loss when labels are given), as run by the fresh inference session of
 * the train-to-deploy example (README "Contents").  x: device float32 [B, d0].  logits: device float32
 * [B, C] or NULL.  labels: device float32 [B, C] (dense, non-negative rows)
 * or NULL.  loss: host float, written (after a stream synchronisation) with
 * the mean softmax cross-entropy when labels and loss are both non-NULL.
 * Without a loss request the call returns once the work is enqueued. */
mlp_status mlp_forward(mlp_ctx* ctx, const float* x, float* logits,
                       const float* labels, float* loss);

/* Forward pass to class probabilities, for inference (the deployed model of
 * the README's train-to-deploy flow): probs[b][c] = exp(z[b][c] - mu_b) /
 * sum_c exp(z[b][c] - mu_b) of the logits z, mu_b = max_c z[b][c] -- the
 * normalisation the loss uses.  x: device float32 [B, d0]; probs: device
 * float32 [B, C], written in stream order (nothing waits).  In strict-f32
 * sessions whose logits product runs on 32 x 16 small-product tiles and
 * C <= 16, the product's epilogue normalises each row itself; otherwise one
 * row-softmax launch follows the forward.  Both pointers must be 16-byte
 * aligned (MLP_ERR_ARG).  The logits kept for mlp_forward are not updated
 * on the fused path. */
mlp_status mlp_forward_probs(mlp_ctx* ctx, const float* x, float* probs);

/* One training step (README "Example": trainer.train, one batch; the
 * autodiff of build_session gives the backward): forward, mean softmax-CE, backward and the update of
 * every layer (W_l <- W_l - lr * dW_l, or the rule mlp_set_optimizer chose),
 * all gradients taken at the pre-update weights.  x: device float32 [B, d0]; labels: device float32
 * [B, C]; lr: finite.  loss: host float or NULL; the call synchronises the
 * stream and writes the mean loss at the pre-update weights. */
mlp_status mlp_train_step(mlp_ctx* ctx, const float* x, const float* labels,
                          float lr, float* loss);

/* Size of the static device buffer of mlp_train_step_static, per GPU. */
#define MLP_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): one SGD
 * training step of a float32 configuration, the computation of
 * mlp_train_step_async, without a context or a workspace.  weights: host
 * array of cfg->n_layers device pointers, each a float32
 * [dims[l], dims[l+1]] weight that the step reads and updates in place.
 * x: device float32 [B, d0]; labels: device float32 [B, C]; lr finite;
 * loss_dev: device float32 or NULL (the mean loss at the pre-update
 * weights, in stream order).  Everything else the step needs lives in a
 * static device array of the library, MLP_STATIC_SCRATCH_BYTES per GPU,
 * held from the library's load on that GPU until the process ends; its
 * address is looked up once per GPU.  Nothing is allocated and nothing
 * waits; the launches go to cfg->stream.  The plan of the last
 * configuration is kept per GPU and rebuilt (host work) when the
 * configuration or stream changes, and the buffer's counters are then
 * cleared by a kernel; every step leaves them cleared again.  All calls on
 * one GPU share that buffer: calls whose work may overlap on the GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 * Errors (checked before anything is enqueued; message in
 * mlp_last_error(NULL)): MLP_ERR_SHAPE / MLP_ERR_ARG as for mlp_create,
 * MLP_ERR_ARG for a bf16 configuration, NULL or misaligned pointers or a
 * non-finite lr, MLP_ERR_WORKSPACE when the configuration needs more than
 * MLP_STATIC_SCRATCH_BYTES, MLP_ERR_ARG when cfg->stream belongs to another
 * device than the current one (the buffer used is the current device's),
 * MLP_ERR_HIP for a failed launch (the weights are then undefined). */
mlp_status mlp_train_step_static(const mlp_config* cfg, float* const* weights, const float* x,
                                 const float* labels, float lr, float* loss_dev);

/* As mlp_train_step, but nothing waits: the mean loss is written to
 * `loss_dev` (device float32, or NULL to drop it) in stream order (README
 * "Debugging" separates a session's step() from its wait()).  Errors as
 * mlp_train_step; a HIP failure after the first launch poisons the
 * context. */
mlp_status mlp_train_step_async(mlp_ctx* ctx, const float* x, const float* labels,
                                float lr, float* loss_dev);

/* n training steps on n successive batches, enqueued without waiting: the
 * loop the README "Example" trainer runs over its data loader's batches.
 * The result is bitwise that of n calls of mlp_train_step_async on the same
 * batches in order.  x: device float32 [n, B, dims[0]] and labels: device
 * float32 [n, B, dims[n_layers]], batch after batch, 16-byte aligned; all of
 * them must stay valid until the stream has run the steps.  loss_dev:
 * device float32 [n] (step s's mean loss at loss_dev[s]) or NULL.  In
 * sessions whose batch has at most 8 rows (the weight-streaming kernels),
 * float32 with SGD, the launch that updates the first layer's weights also
 * computes the next step's first-layer forward from the updated values, so
 * each step after the first makes one pass fewer over that matrix; per-launch
 * timing (mlp_profile_enable) records none of such a run's steps.  Errors
 * as mlp_train_step_async, and MLP_ERR_ARG for n < 1 or, when n > 1, a
 * batch whose x or labels size is not a multiple of 16 bytes (later batches
 * would lose the alignment); a HIP failure poisons the context and leaves
 * the weights undefined. */
mlp_status mlp_train_steps(mlp_ctx* ctx, int32_t n, const float* x, const float* labels,
                           float lr, float* loss_dev);

/* Gradients without an update, from the same kernels and accumulation order
 * as a training step: the backward of README "Example" read out as a debug
 * session would (README "Debugging"), so that forward and backward can be
 * gated separately (arXiv abstract of "Meganeura: Portable GPU Training and
 * Inference through Vulkan and Metal").  dw: host array of n_layers device pointers, each a
 * float32 [dims[l], dims[l+1]] output.  dlogits: device float32 [B, C] or
 * NULL.  loss: host float or NULL (the call synchronises when non-NULL). */
mlp_status mlp_grads(mlp_ctx* ctx, const float* x, const float* labels,
                     float* const* dw, float* dlogits, float* loss);

/* Device memory (bytes, a multiple of 256) that update rule `opt` keeps for
 * this configuration: float32 first and second moments per weight.  0 for
 * MLP_OPT_SGD, for an unknown rule and for an invalid configuration.  Host
 * only. */
size_t mlp_optimizer_bytes(const mlp_config* cfg, int32_t opt);

/* Select the update rule of mlp_train_step / mlp_train_step_async (the
 * default is MLP_OPT_SGD).  For Adam and LaProp, `state` is caller-owned
 * device memory of at least mlp_optimizer_bytes(cfg, opt) bytes, 256-byte
 * aligned, that must stay alive while the rule is in use; both moments are
 * zeroed (enqueued on the context's stream) and the step count t restarts,
 * so the next step has t = 1.  beta1, beta2 in [0, 1); eps finite and > 0.
 * For SGD, state, bytes, beta1, beta2 and eps are ignored.  Every dW launch
 * applies the rule while it holds W (reading and writing W, m and v once);
 * the step count is a launch argument, so such steps refuse (MLP_ERR_ARG)
 * to be enqueued while the stream is being captured.  Errors:
 * MLP_ERR_ARG (rule, betas, eps), MLP_ERR_WORKSPACE (state), MLP_ERR_STATE
 * (poisoned context); nothing changes on an error.  Resets the per-launch
 * timing (the launch sequence changes). */
mlp_status mlp_set_optimizer(mlp_ctx* ctx, int32_t opt, float beta1, float beta2, float eps,
                             void* state, size_t bytes);

/* Checkpoints (README "Contents": tensors are stored at their logical
 * shapes without the device's padding, and a restore is validated in full
 * before it changes any state; the train-to-deploy example reloads one into
 * a fresh inference session).
 * A checkpoint is host memory: a 136-byte header (magic "MLPCKPT1", version
 * 2, layer count, precision of the writer, update rule, widths, beta1, beta2,
 * eps, step count, payload size, checksum of the payload) and the
 * payload: every W_l as float32 [dims[l], dims[l+1]] row-major, then, when
 * the rule's state is included, every m_l and every v_l in the same shapes.
 * Little-endian; the header's fields are, in order and without padding:
 * char magic[8], uint32 version, n_layers, precision, optimizer, int32
 * dims[17] (n_layers+1 used, the rest 0), float beta1, beta2, eps, uint32
 * reserved[2] (0), int64 step, uint64 payload_bytes, uint64 checksum.
 * Checksum: with FNV-1a-64's offset basis B = 0xcbf29ce484222325 and prime
 * P = 0x100000001b3, the payload is read as little-endian uint64 words (a
 * final 4-byte remainder zero-extended to a word); word i is folded into lane
 * i mod 4, h = (h XOR word) * P mod 2^64, every lane starting at B; the
 * checksum is byte-wise FNV-1a-64 (r = B; per byte r = (r XOR byte) * P) over
 * the 32 little-endian bytes of lanes 0, 1, 2, 3.  Version 1 checkpoints
 * (another checksum) are refused. */

/* Size of the checkpoint mlp_save_checkpoint writes; with_optimizer != 0
 * includes the Adam/LaProp moments when the session uses such a rule.
 * 0 for ctx == NULL. */
size_t mlp_checkpoint_bytes(const mlp_ctx* ctx, int32_t with_optimizer);

/* Write the checkpoint of the current weights (and moments) into host
 * memory `dst` of at least mlp_checkpoint_bytes bytes.  Synchronises the
 * context's stream first, so the state after every enqueued step is saved.
 * MLP_ERR_STATE if the weights were never set or the context is poisoned. */
mlp_status mlp_save_checkpoint(mlp_ctx* ctx, void* dst, size_t bytes, int32_t with_optimizer);

/* Check a checkpoint in host memory without a context (no device work):
 * magic, version, ranges, payload size and checksum.  On success writes the
 * layer count, the n_layers+1 widths (dims: room for 17), the update rule
 * whose state it carries (MLP_OPT_SGD: none) and its step count, each when
 * the pointer is non-NULL.  Errors: MLP_ERR_ARG, message in
 * mlp_last_error(NULL). */
mlp_status mlp_checkpoint_info(const void* src, size_t bytes, int32_t* n_layers, int32_t* dims,
                               int32_t* optimizer, int64_t* step);

/* Restore weights (and moments) from a checkpoint in host memory.  Preflight
 * before anything is written: the checks of mlp_checkpoint_info, the same
 * layer count and widths as the session (MLP_ERR_SHAPE otherwise), and, for
 * a session using Adam/LaProp, the same rule, betas and eps with its state
 * in the checkpoint (MLP_ERR_ARG otherwise); on any of these errors nothing
 * changes.  A session on SGD restores the weights only (a forward-only or
 * SGD session may load a checkpoint written with moments).  The bf16
 * operand copies are rebuilt; the step count of the moments is restored.
 * The precision of the writer does not matter (masters are float32).
 * Synchronises the context's stream before returning. */
mlp_status mlp_load_checkpoint(mlp_ctx* ctx, const void* src, size_t bytes);

/* Choose launch plans by measurement (README "Contents": MEGANEURA_TUNE and
 * tune_with, a bounded per-shape search): for every product of the step, the
 * tile shape and K split among a small fixed set, each timed over `repeats`
 * steps (1..100) on this batch (device x [B, d0], labels [B, C]) with
 * per-launch events; a candidate replaces the current plan only when the
 * step gets at least 2% faster.  The timed steps use SGD with lr = 0, so
 * finite weights and any optimizer state are unchanged.  Candidates stay
 * within the workspace planned at creation; the plans the fused output
 * layer depends on are kept.  Skinny-batch sessions (batch <= 16) choose the
 * K split of each forward pass and the column split of each fused dX + dW
 * pass instead.  Synchronises the stream.  A tuned context stays deterministic
 * from step to step, but its sums may be ordered differently from an
 * untuned one (other tile shapes or K splits).  Refuses stream capture. */
mlp_status mlp_tune(mlp_ctx* ctx, const float* x, const float* labels, int32_t repeats);

/* Copy an intermediate of the last step or forward to device memory `dst`
 * (see mlp_state_kind for shapes; `layer` is 1..n_layers-1 for ACT/MASK). */
mlp_status mlp_read_state(mlp_ctx* ctx, int32_t which, int32_t layer, void* dst);

/* Per-launch timing.  When enabled, every kernel launch of a step is
 * bracketed by a pair of HIP events on the context's stream (the README's
 * per-dispatch GPU timing).  mlp_profile_read sums the recorded durations
 * per launch slot after the caller has synchronised the stream.  Training
 * steps (and mlp_grads), forward passes and forward passes with a loss are
 * three launch sequences with slots of their own; the slot calls below
 * report the sequence of the last call enqueued while timing was enabled. */
mlp_status mlp_profile_enable(mlp_ctx* ctx, int32_t enable);
mlp_status mlp_profile_reset(mlp_ctx* ctx);
/* Number of launch slots in that sequence. */
int32_t mlp_profile_slots(const mlp_ctx* ctx);
/* Slot `idx`: slot name (the launch's products, copied into `name`,
 * NUL-terminated), total
 * milliseconds and launch count since the last reset, and the slot's
 * algorithmic flops and HBM bytes per launch. */
mlp_status mlp_profile_read(mlp_ctx* ctx, int32_t idx, char* name, size_t name_len,
                            double* total_ms, int64_t* launches,
                            double* flops, double* bytes);

/* Debug modes (README "Environment variables": MEGANEURA_SERIAL_DISPATCH
 * runs one dispatch at a time to bisect a failure, MEGANEURA_PIN_BUFS pins
 * buffers to bisect aliasing corruption; README "Debugging": failures come
 * back as structured errors that name what went wrong).
 *   MLP_DEBUG_SYNC   -- after every kernel launch the stream is synchronised,
 *                       so a HIP error that shows only at execution is
 *                       reported (MLP_ERR_HIP) with the name of that launch
 *                       (the profile slot name) in mlp_last_error.  Launch
 *                       errors name their launch in every mode.
 *   MLP_DEBUG_GUARDS -- after every call that runs kernels (mlp_forward,
 *                       mlp_forward_probs, mlp_train_step[_async],
 *                       mlp_train_steps, mlp_grads, mlp_tune) the stream is
 *                       synchronised and every guard band of the workspace
 *                       is compared with the pattern mlp_create wrote there
 *                       (bytes 0xA5).  A changed band means a write past the
 *                       end of the buffer before it: the call returns
 *                       MLP_ERR_GUARD, mlp_last_error names the buffer and
 *                       the first changed byte, the bands are rewritten and
 *                       the context is poisoned as after a HIP failure (the
 *                       weights may be damaged; mlp_set_params or
 *                       mlp_load_checkpoint for every layer clears it).
 * Both make the calls above wait for the device, and neither applies while
 * the stream is being captured into a graph.  The checks are host work
 * outside the kernels, so a step's results are the same in every mode. */
typedef enum mlp_debug_flags {
    MLP_DEBUG_SYNC = 1,
    MLP_DEBUG_GUARDS = 2
} mlp_debug_flags;

/* Set the debug modes (an OR of mlp_debug_flags; 0 = off, the default).
 * Errors: MLP_ERR_ARG for a NULL context or unknown bits. */
mlp_status mlp_set_debug(mlp_ctx* ctx, int32_t flags);

/* Name of a status code ("MLP_OK", ...; "MLP_ERR_UNKNOWN" otherwise), a
 * static string.  With mlp_last_error, the structured errors of README
 * "Debugging". */
const char* mlp_status_string(mlp_status s);
/* Message of the last error on this context ("" if none); valid until the
 * next call on the context.  With ctx == NULL: the last creation error (or
 * checkpoint_info error) of this thread.  README "Debugging": failures come
 * back as structured errors that name what went wrong. */
const char* mlp_last_error(const mlp_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* MLP_H_ */
