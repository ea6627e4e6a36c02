/*
 * gpt2.h - C ABI of libgpt2.so: one GPT-2 training step on an MI355X (gfx950).
 *
 * The library computes, on one GPU, what a PyTorch GPT-2 training step
 * computes ("GPT-2 from Scratch", sections "The full model", "The loop",
 * "How to scale up"; "Let's reproduce GPT-2 (124M)", optimizer and
 * accumulation paragraphs):
 *
 *   loss   = gpt2_forward(idx, targets)       model(idx, targets) -> mean CE
 *            gpt2_backward(loss_scale)        (loss * loss_scale).backward()
 *   norm   = gpt2_adamw_step(lr, ...)         clip_grad_norm_(params, max) + AdamW.step()
 *
 * Model: pre-LayerNorm decoder-only transformer with learned positions,
 * fused qkv projection, causal softmax attention, GELU (tanh form) MLP of
 * width 4C, final LayerNorm, lm_head tied to the token embedding, padded
 * vocabulary.  Cross-entropy ignores targets equal to -1 and averages over
 * the remaining positions.
 *
 * Memory.  The caller allocates ONE device buffer (the workspace) of
 * gpt2_workspace_bytes() bytes and keeps it alive until gpt2_destroy.  The
 * library never allocates device memory; parameters, gradients, AdamW
 * moments, the bf16 weight copy, saved activations and scratch all live in
 * the workspace at offsets the library chooses.
 *
 * Streams.  Every call enqueues its work on the HIP stream given to
 * gpt2_init (hipStream_t passed as void*; NULL is the default stream) and
 * returns without waiting, except where a host output pointer is given
 * (h_loss, h_grad_norm, host copies), in which case it waits for the stream.
 * A handle must not be used from two threads at once.
 *
 * Errors.  Every call returns a gpt2_status; nothing aborts.  Argument and
 * shape errors are detected on the host before anything is enqueued.  Token
 * ids outside [0, padded_vocab_size) and targets outside
 * {-1} U [0, padded_vocab_size) are detected on the device: the kernels clamp
 * the offending read so nothing faults, set a device flag, and the next
 * synchronising call (gpt2_sync, or any call given a host output) returns
 * GPT2_E_RANGE.  gpt2_last_error() gives a human-readable message.
 *
 * Precision.  GPT2_FP32: every tensor and every product in fp32.
 * GPT2_BF16: matrix products (the five linear layers and attention) take
 * bf16 operands rounded to nearest-even from fp32 and accumulate in fp32;
 * the residual stream, LayerNorm statistics, softmax, cross-entropy,
 * gradients of parameters, master weights and AdamW state are fp32; other
 * saved activations (LayerNorm outputs, qkv, attention output, MLP hidden,
 * logits) are stored in bf16.  This is the placement torch.autocast with
 * bfloat16 gives ("Let's reproduce GPT-2 (124M)", precision paragraph).
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT2_OK = 0,
  GPT2_E_ARG = -1,    /* bad argument: NULL pointer, size mismatch, unsupported config */
  GPT2_E_SHAPE = -2,  /* B < 1, B > max_batch, T < 1 or T > block_size */
  GPT2_E_RANGE = -3,  /* a token id or target was out of range (device-detected) */
  GPT2_E_STATE = -4,  /* call order violated (backward without a forward with targets) */
  GPT2_E_HIP = -5     /* a HIP runtime call failed; see gpt2_last_error */
} gpt2_status;

typedef enum { GPT2_FP32 = 0, GPT2_BF16 = 1 } gpt2_precision;

/* Model and capacity.  n_embd % n_head == 0.  In GPT2_BF16 the head width
 * n_embd / n_head must be 64 (every released GPT-2 size, "The config");
 * GPT2_FP32 accepts head widths 32 and 64.  n_embd must be a multiple of 64
 * and padded_vocab_size a multiple of 64 and >= vocab_size.  max_batch
 * bounds B for the activation storage. */
typedef struct {
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;
  int32_t vocab_size;
  int32_t padded_vocab_size;
  int32_t block_size;
  int32_t max_batch;
  int32_t precision; /* gpt2_precision */
  /* 0: the lm_head writes the (B*T, padded_vocab_size) logits and the
   * cross-entropy turns them into their gradient in place.  > 0 (a multiple
   * of 64): fused lm_head + cross-entropy that never stores those logits.
   * The forward's GEMM epilogue reduces each row's logits to log-sum-exp
   * partials over 64-column blocks and picks out the target's logit; the
   * backward recomputes the logits slice by slice, head_chunk vocabulary
   * columns at a time, turns each slice into its gradient in the epilogue
   * and applies it to dz and dwte.  Same results up to rounding ("Let's
   * reproduce GPT-2 (124M)", the remark on the fp32 logits tensor of the
   * loss); one more (B*T, C, Vp) product per step; the workspace holds one
   * (B*T, head_chunk) slice instead of the logits.  With a fused head a
   * forward without targets stops after the final LayerNorm and
   * GPT2_ACT_LOGITS is not available. */
  int32_t head_chunk;
} gpt2_config;

typedef struct gpt2 gpt2_t; /* opaque handle */

/* Number of parameters with the tied embedding counted once, in the
 * canonical order used by gpt2_set_params/gpt2_get:
 *   wte (Vp, C); wpe (block_size, C);
 *   per layer: ln_1.w (C), ln_1.b (C), c_attn.w (3C, C), c_attn.b (3C),
 *              attn c_proj.w (C, C), attn c_proj.b (C), ln_2.w (C), ln_2.b (C),
 *              c_fc.w (4C, C), c_fc.b (4C), mlp c_proj.w (C, 4C), mlp c_proj.b (C);
 *   ln_f.w (C), ln_f.b (C).
 * Matrices are row-major (out, in) as for a torch Linear.  ("GPT-2 from
 * Scratch": "Embeddings", "CausalSelfAttention", "The MLP", "The Block",
 * "Weight tying".)  Returns 0 for an invalid config. */
size_t gpt2_num_params(const gpt2_config* cfg);

/* Bytes of device workspace a handle needs for this config. */
gpt2_status gpt2_workspace_bytes(const gpt2_config* cfg, size_t* bytes);

/* Creates a handle over a caller-owned device workspace (256-byte aligned,
 * at least gpt2_workspace_bytes) and initialises the parameters on the device
 * from `seed` ("GPT-2 from Scratch", Initialization: 0.02, and the residual
 * scaling): every weight matrix and both embeddings N(0, 0.02), the two
 * c_proj weights of each block N(0, 0.02 / sqrt(2 n_layer)), biases and
 * LayerNorm shifts 0, LayerNorm gains 1.  The normal numbers are a stream
 * fixed by the seed alone: element e of the canonical vector (see
 * gpt2_num_params) takes number e, produced by the counter-based generator
 * Philox4x32-10 (Salmon et al., SC 2011) on counter (e/4 mod 2^32, e/4 / 2^32,
 * 0, 0) and key (seed mod 2^32, seed / 2^32), its four words turned into
 * uniforms (floor(x / 2^9) + 1/2) / 2^23 and two Box-Muller pairs (element
 * 4b + j takes pair j/2's cosine (j even) or sine (j odd) branch).  Gradients
 * and AdamW moments start at zero, the step count at 0.  gpt2_set_params
 * replaces the parameters.  hip_stream: the hipStream_t to use.  On any
 * failure *out is NULL; nothing is left allocated. */
gpt2_status gpt2_init(const gpt2_config* cfg, void* d_workspace, size_t ws_bytes,
                      void* hip_stream, uint64_t seed, gpt2_t** out);

/* Loads all parameters (fp32, canonical order, n == gpt2_num_params) from
 * host (src_on_device = 0) or device memory, refreshes the bf16 weight copy,
 * zeroes the AdamW moments and gradients, and resets the step count to 0. */
gpt2_status gpt2_set_params(gpt2_t* h, const float* src, size_t n, int src_on_device);

enum { GPT2_PARAMS = 0, GPT2_GRADS = 1, GPT2_ADAM_M = 2, GPT2_ADAM_V = 3 };

/* Copies one fp32 state vector (canonical order, n == gpt2_num_params) to
 * host or device memory.  Host copies wait for the stream. */
gpt2_status gpt2_get(gpt2_t* h, int which, float* dst, size_t n, int dst_on_device);

/* Overwrites one state vector (GRADS, ADAM_M or ADAM_V; PARAMS goes through
 * gpt2_set_params) without other side effects.  Used to resume. */
gpt2_status gpt2_set_state(gpt2_t* h, int which, const float* src, size_t n, int src_on_device);

/* AdamW step counter t (number of gpt2_adamw_step calls since set_params). */
gpt2_status gpt2_get_step(const gpt2_t* h, int64_t* t);
gpt2_status gpt2_set_step(gpt2_t* h, int64_t t);

/* Learning rate of optimizer step `step` (0-based), for the caller to pass
 * to gpt2_adamw_step ("GPT-2 from Scratch", Warmup and cosine decay; the
 * pretraining recipe of "Pretraining and fine-tuning nanoGPT-124M" uses
 * eta_max 6e-4, eta_min 6e-5, 715 warmup steps): a linear ramp
 * eta_max (step + 1) / warmup_steps while step < warmup_steps; then
 * eta_min + (eta_max - eta_min) (1 + cos(pi s)) / 2 with
 * s = (step - warmup_steps) / (max_steps - warmup_steps) (s = 0 when the two
 * are equal) up to step == max_steps; eta_min after.  Host arithmetic in
 * double, nothing is enqueued.  GPT2_E_ARG if lr is NULL, step < 0,
 * warmup_steps < 1 or max_steps < warmup_steps. */
gpt2_status gpt2_lr_at(int64_t step, double eta_max, double eta_min, int64_t warmup_steps,
                       int64_t max_steps, double* lr);

/* Forward pass over a batch: d_idx, d_targets are device int32 arrays of B*T
 * ids, row-major (B, T); targets[b][t] is the id that should follow
 * idx[b][t], or -1 to leave the position out of the loss.  d_targets may be
 * NULL: then only logits are computed (read them with gpt2_get_activation).
 * With targets, the loss is the mean of -log softmax(logits)[target] over
 * positions with target != -1 (0 if there are none), and the gradient of
 * the loss with respect to the logits is formed in the same pass, in place of
 * the logits, ready for gpt2_backward.  If h_loss is non-NULL the call waits
 * and stores the loss there.  Both arrays are read before the call's work
 * completes on the stream; the ids are copied into the workspace for the
 * backward pass. */
gpt2_status gpt2_forward(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets,
                         int B, int T, float* h_loss);

/* Evaluation pass ("Measuring held-out loss"; per-sequence scoring of
 * candidate continuations, as multiple-choice evaluations do): the forward
 * pass and the cross-entropy losses only -- no gradient is formed, the logits
 * stay in place (gpt2_get_activation LOGITS) and a following gpt2_backward
 * returns GPT2_E_STATE.  d_targets is required (device int32, B*T, -1 =
 * ignored).  d_seq_loss (device, B floats, may be NULL) receives for each
 * sequence b the mean loss over its positions with a target,
 *   sum_t loss[b][t] / #{t : targets[b][t] != -1}   (0 if there is none),
 * and h_loss (host, may be NULL; waits) the mean over all such positions of
 * the batch, exactly what gpt2_forward would report. */
gpt2_status gpt2_eval(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, int B, int T,
                      float* d_seq_loss, float* h_loss);

/* Generation ("GPT-2 from Scratch", The full model: without targets only
 * the last position goes through the lm_head; A generation loop).
 *
 * gpt2_forward_last: forward pass over (B, T) ids with no targets; writes the
 * lm_head output of the last position of each sequence, d_logits (device,
 * fp32, (B, padded_vocab_size) row-major).  Activations of the pass stay
 * readable; a following gpt2_backward returns GPT2_E_STATE. */
gpt2_status gpt2_forward_last(gpt2_t* h, const int32_t* d_idx, int B, int T, float* d_logits);

/* One draw per row of d_logits (device fp32, B rows of V entries at a row
 * stride of ld floats; ld % 4 == 0, 16-byte aligned, V <= 53248):
 *   x = logits / temperature (temperature > 0);
 *   top_k > 0 and < V: entries below the k-th largest x are dropped (entries
 *   equal to it stay); top_k <= 0 keeps all;
 *   p = softmax(x) over the entries kept;
 *   d_tokens[b] (device int32) = the smallest i whose cumulative probability
 *   exceeds d_uniform[b] (device fp32, a uniform in [0, 1) per row supplied by
 *   the caller: the multinomial draw as an inverse CDF over the entries in
 *   index order); if rounding leaves none, the last entry kept.
 * The k-th largest value is selected exactly; the sums are fp32 in a fixed
 * order, so equal inputs give equal tokens. */
gpt2_status gpt2_sample(gpt2_t* h, const float* d_logits, long ld, int B, int V, float temperature,
                        int top_k, const float* d_uniform, int32_t* d_tokens);

/* The sampling loop: d_out (device int32, (B, T0 + n_new) row-major) gets the
 * prompt d_prompt (device int32, (B, T0)) followed by n_new drawn tokens.
 * Step s crops each running sequence to its last block_size tokens, runs
 * gpt2_forward_last on them and draws with gpt2_sample's rule over the
 * padded vocabulary, using d_uniform[b * n_new + s] (device fp32, (B, n_new)).
 * Each step recomputes the whole cropped context (no key/value cache).
 * Asynchronous: nothing waits; out-of-range prompt ids are reported by the
 * next synchronising call.  Saved activations are not readable afterwards. */
gpt2_status gpt2_generate(gpt2_t* h, const int32_t* d_prompt, int B, int T0, int n_new,
                          float temperature, int top_k, const float* d_uniform, int32_t* d_out);

/* gpt2_generate with a key/value cache ("GPT-2 from Scratch", A generation
 * loop: recomputing the whole context for every new token is the quadratic
 * cost a key/value cache removes).  Same arguments, the same draws up to the
 * rounding of the products: the prompt's keys and values of every block are
 * computed once, by one forward pass over (B, T0), and kept in the
 * workspace; each new token then runs the blocks for its own position only,
 * its attention reading the kept keys and values of the positions before it
 * and adding its own.  Once a sequence has reached block_size tokens, every
 * later step crops the window, which moves every position embedding, so
 * those steps recompute the cropped window as gpt2_generate does (and a
 * prompt longer than block_size is recomputed from the first step).
 * GPT2_E_ARG if block_size > 8192.  Asynchronous like gpt2_generate;
 * saved activations are not readable afterwards. */
gpt2_status gpt2_generate_cached(gpt2_t* h, const int32_t* d_prompt, int B, int T0, int n_new,
                                 float temperature, int top_k, const float* d_uniform,
                                 int32_t* d_out);

/* The key/value-cached decoding of gpt2_generate_cached, one position per
 * call, for callers that draw the tokens themselves ("GPT-2 from Scratch",
 * A generation loop: the logits of the last position of each running
 * sequence are what the loop samples from).
 *
 * gpt2_prefill runs the blocks over d_idx (device int32, (B, T) row-major,
 * 1 <= B <= max_batch, 1 <= T <= block_size), keeps every block's keys and
 * values of positions 0 .. T-1 in the workspace, and writes the logits of
 * position T-1 of each sequence to d_logits (device fp32, (B, padded
 * vocabulary) row-major, 16-byte aligned; entries past vocab_size are the
 * products with the zero rows of the padded embedding).
 *
 * gpt2_decode takes d_tok (device int32, (B)), the token at position p of
 * each sequence, where p is the number of positions already kept (the T of
 * the last gpt2_prefill plus the gpt2_decode calls since) and B the batch of
 * that gpt2_prefill; it runs the blocks for position p only, its attention
 * reading the kept keys and values of positions 0 .. p-1 and keeping those
 * of p, and writes the logits of position p to d_logits as above.
 *
 * Errors: GPT2_E_ARG for null or misaligned pointers (and block_size >
 * 8192); GPT2_E_SHAPE for B or T out of range, or p = block_size (the cache
 * is full); GPT2_E_STATE for a gpt2_decode that does not continue the kept
 * sequences (no gpt2_prefill yet, another B or p; also after
 * gpt2_set_params, gpt2_adamw_step or gpt2_generate_cached, which leave the
 * kept keys and values stale).  Asynchronous: out-of-range token ids are
 * reported by the next synchronising call.  Saved activations are not
 * readable afterwards. */
gpt2_status gpt2_prefill(gpt2_t* h, const int32_t* d_idx, int B, int T, float* d_logits);
gpt2_status gpt2_decode(gpt2_t* h, const int32_t* d_tok, int B, int p, float* d_logits);

/* Loss of the last forward with targets; waits for the stream. */
gpt2_status gpt2_get_loss(gpt2_t* h, float* h_loss);

/* Sets every gradient to zero.  Deferred: the next backward then writes the
 * gradients it produces instead of adding them where it writes each one
 * whole (bf16 with B*T a multiple of 64), and any
 * other use of the gradients (gpt2_get, gpt2_adamw_step, a backward that
 * adds) zeroes them first; the result is the same. */
gpt2_status gpt2_zero_grad(gpt2_t* h);

/* Backward pass of the last forward with targets: adds loss_scale *
 * d(loss)/d(param) into the gradients (use loss_scale = 1/k for k
 * accumulation micro-steps, "How to scale up").  The tied embedding gets the
 * sum of its lm_head and embedding contributions.  GPT2_E_STATE if the last
 * forward had no targets or a backward already consumed it. */
gpt2_status gpt2_backward(gpt2_t* h, float loss_scale);

/* Global-norm clip and AdamW ("Gradient clipping"; "AdamW, and weight decay
 * on matrices only"): norm = ||g||_2 over all parameters; g is scaled by
 * min(1, max_grad_norm / (norm + 1e-6)); then, per element, with t the
 * updated step count (1 on the first call):
 *   p <- p * (1 - lr * weight_decay)   only for tensors with dim >= 2
 *   m <- beta1 m + (1 - beta1) g ;  v <- beta2 v + (1 - beta2) g^2
 *   p <- p - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 * The bf16 weight copy is refreshed.  Gradients are left unchanged (not
 * clipped in place).  If h_grad_norm is non-NULL the call waits and stores
 * the pre-clip norm there. */
gpt2_status gpt2_adamw_step(gpt2_t* h, float lr, float beta1, float beta2, float eps,
                            float weight_decay, float max_grad_norm, float* h_grad_norm);

/* Pre-clip gradient norm of the last gpt2_adamw_step; waits. */
gpt2_status gpt2_get_grad_norm(gpt2_t* h, float* h_norm);

/* Waits for the stream and reports device-side errors (GPT2_E_RANGE). */
gpt2_status gpt2_sync(gpt2_t* h);

/* Message describing the last error on this handle ("" if none). */
const char* gpt2_last_error(const gpt2_t* h);

/* Releases the handle (not the workspace, which the caller owns). */
void gpt2_destroy(gpt2_t* h);

/* Saved activations of the last forward, for layer-by-layer comparison
 * against a reference.  `layer` selects the block where it applies.  The
 * tensor is converted to fp32 and copied to host memory (waits).  The first
 * n elements (row-major) are copied; n may not exceed the element count given
 * for each id below (B, T of the last forward):
 *   X_IN      residual stream entering block `layer` (layer == n_layer: after the last block), B*T*C
 *   LN1       ln_1 output, B*T*C          QKV    c_attn output, B*T*3C ([q | k | v])
 *   ATTN_Y    attention output with heads re-interleaved, B*T*C
 *   LSE       per (b, head, t) log-sum-exp of the scaled, masked scores, B*H*T
 *   X_MID     residual stream after attention, B*T*C
 *   LN2       ln_2 output, B*T*C
 *   FC_DGELU  GELU derivative at the c_fc output, gelu'(h) (saved for the backward), B*T*4C
 *   FC_GELU   GELU output, B*T*4C         LNF     ln_f output, B*T*C
 *   LOGITS    logits (forward without targets) or, after a forward with
 *             targets, d(loss)/d(logits) which replaces them, B*T*Vp
 *   ROW_LOSS  per-position loss (0 where target == -1), B*T */
enum {
  GPT2_ACT_X_IN = 0, GPT2_ACT_LN1, GPT2_ACT_QKV, GPT2_ACT_ATTN_Y, GPT2_ACT_LSE, GPT2_ACT_X_MID,
  GPT2_ACT_LN2, GPT2_ACT_FC_DGELU, GPT2_ACT_FC_GELU, GPT2_ACT_LNF, GPT2_ACT_LOGITS,
  GPT2_ACT_ROW_LOSS
};
gpt2_status gpt2_get_activation(gpt2_t* h, int which, int layer, float* h_dst, size_t n);

/* Kernel timing.  Launch sites of the step, for per-kernel measurement with
 * HIP events recorded on the handle's stream around each launch.  With a
 * fused head (head_chunk > 0) LMHEAD_FWD is the partials GEMM, XENT the
 * log-sum-exp and loss reduction, LMHEAD_RECOMP the backward's recomputation
 * of a slice of logits, LMHEAD_DX/DW the slices' shares of dz and dwte.
 * ADAMW covers the optimizer update: in GPT2_BF16 one launch over 64 x 64
 * tiles of the matrices that the input-gradient products read transposed
 * (it also writes their bf16 and transposed bf16 copies) and one over every
 * other tensor.  WEIGHT_T is kept for the numbering and records nothing.
 * In GPT2_BF16 with
 * B*T a multiple of 64, the weight gradients of all blocks (and of the
 * lm_head, unless fused) run as one grouped launch at the end of the
 * backward pass, timed as WGRAD; the per-product *_DW sites are then empty.
 * When the group's tile count would leave the last round of the launch mostly
 * idle, the first product's last tile-rows are taken out of the group and run
 * afterwards as a small split-K product, timed as WGRAD_TAIL. */
enum {
  GPT2_SITE_EMBED_FWD = 0, GPT2_SITE_LN_FWD, GPT2_SITE_QKV_FWD, GPT2_SITE_ATTN_FWD,
  GPT2_SITE_PROJ_FWD, GPT2_SITE_FC_FWD, GPT2_SITE_FCPROJ_FWD, GPT2_SITE_LMHEAD_FWD,
  GPT2_SITE_XENT, GPT2_SITE_LMHEAD_DX, GPT2_SITE_LMHEAD_DW, GPT2_SITE_LN_BWD,
  GPT2_SITE_FCPROJ_DX, GPT2_SITE_FCPROJ_DW, GPT2_SITE_FC_DX, GPT2_SITE_FC_DW,
  GPT2_SITE_PROJ_DX, GPT2_SITE_PROJ_DW, GPT2_SITE_ATTN_BWD, GPT2_SITE_QKV_DX,
  GPT2_SITE_QKV_DW, GPT2_SITE_BIAS_GRAD, GPT2_SITE_EMBED_BWD, GPT2_SITE_GRAD_NORM,
  GPT2_SITE_ADAMW, GPT2_SITE_ZERO_GRAD, GPT2_SITE_LMHEAD_RECOMP, GPT2_SITE_WEIGHT_T,
  GPT2_SITE_WGRAD, GPT2_SITE_WGRAD_TAIL, GPT2_NUM_SITES
};

/* From now on, record an event pair around every launch of each site whose
 * bit is set in site_mask (bit i = site i).  Clears earlier records.  Event
 * objects are created on first use and kept for later sessions. */
gpt2_status gpt2_timing_begin(gpt2_t* h, uint64_t site_mask);

/* Stops recording, waits for the stream, and returns per site the summed
 * duration in milliseconds (ms[GPT2_NUM_SITES]) and the number of launches
 * (launches[GPT2_NUM_SITES]); either pointer may be NULL. */
gpt2_status gpt2_timing_end(gpt2_t* h, double* ms, int32_t* launches);

/* How the backward launches its weight gradients (fixed at gpt2_init, the
 * same for every B, T): the number of weight-matrix gradient elements that
 * the grouped launch (site WGRAD) produces, the number that the split-K tail
 * (site WGRAD_TAIL) produces, and the grouped launch's 256x256 output tiles.
 * Each element is a dot product over the B*T positions, so a launch's matrix
 * work is 2*B*T times its element count.  All three are 0 when the weight
 * gradients run one product at a time (GPT2_FP32; in GPT2_BF16 also any
 * backward whose B*T is not a multiple of 64, which ignores this layout).  Any pointer may be NULL;
 * h NULL returns GPT2_E_ARG. */
gpt2_status gpt2_wgrad_layout(const gpt2_t* h, int64_t* grouped_elems, int64_t* tail_elems,
                              int64_t* grouped_tiles);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_H */
