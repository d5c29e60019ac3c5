/*
 * gpt2.h - C ABI of the MI355X (gfx950) GPT-2 training-step library.
 *
 * One training step of the decoder-only model that the minigpt page
 * ("从零实现一个最小GPT：代码讲解 + 知识点全解", sections 二 and 三) defines:
 * token + position embedding (3.7), pre-LayerNorm blocks (3.6) with fused QKV
 * (the QKV concatenation the karpathy page "两小时手搓GPT-2" raises), causal
 * scaled-dot-product softmax attention (3.3, 3.4), a 4x MLP (3.5) with the tanh
 * approximation of GELU (karpathy page, section on Attention/MLP/GELU), residual
 * adds, a final LayerNorm, a head tied to the token embedding, mean cross-entropy
 * (3.7), the backward pass, and AdamW (3.9). The flat parameter / gradient /
 * activation buffers follow the single-allocation idea the llm.c page
 * ("手写训练脚本", section 二) describes; the layout itself is this library's.
 *
 * Conventions
 *  - Every pointer named d_* or inside gpt2_buffers is DEVICE memory that the
 *    caller allocates and owns (e.g. torch.empty(..., device="cuda")). The
 *    library never allocates, frees or retains device memory beyond the
 *    lifetime of a gpt2_ctx, which only borrows the pointers.
 *  - Every compute call is enqueue-only on the hipStream_t given to gpt2_init
 *    (passed as void*). Scalars it produces (loss, grad norm, argmax) stay in
 *    device memory until the caller copies them.
 *  - Return value: GPT2_OK (0) or a negative GPT2_E* code. Arguments are
 *    validated before anything is enqueued, so an error return leaves device
 *    state unchanged (except GPT2_EHIP, a failed launch).
 *  - Conditions only the device can see (token id outside [0, V), non-finite
 *    loss or gradient norm) set bits of a sticky status word that
 *    gpt2_sync_status reads; they never fault.
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
#define GPT2_OK 0
#define GPT2_EINVAL (-1)   /* bad config / size / null pointer (C % H != 0, T > block_size, ...) */
#define GPT2_ENOSPC (-2)   /* arena smaller than gpt2_query_sizes asked for */
#define GPT2_EHIP (-3)     /* a HIP launch or runtime call failed */
#define GPT2_EDEVICE (-4)  /* gpt2_sync_status: a device status bit is set */
#define GPT2_ESTATE (-5)   /* call out of order (backward without a training forward, ...) */

#define GPT2_DTYPE_F32 0   /* every activation and GEMM/attention operand in fp32 */
#define GPT2_DTYPE_BF16 1  /* bf16 GEMM/attention operands, fp32 accumulation, statistics,
                              residual stream, loss, gradients and optimizer state */

#define GPT2_MODE_TRAIN 0  /* forward keeps what backward needs */
#define GPT2_MODE_EVAL 1   /* forward and loss only; smaller arena */
#define GPT2_MODE_GENERATE 2  /* gpt2_generate only: key/value caches of block_size positions
                                 for B sequences (T must equal block_size) */

#define GPT2_STATUS_TOKEN_RANGE 1u      /* an input or target id was outside [0, V) */
#define GPT2_STATUS_NONFINITE_LOSS 2u   /* the mean loss was NaN or Inf */
#define GPT2_STATUS_NONFINITE_GNORM 4u  /* the global gradient norm was NaN or Inf */
#define GPT2_STATUS_WINDOW_RANGE 8u     /* gpt2_batch_windows: a window start outside [0, n - T - 1] */

/* ------------------------------------------------------------------ types */
/* Model shape (GPTConfig of the minigpt page, section 3.1; the 124M values of
 * train_gpt2.py on the nanogpt page "4.1 GPT-2 124M 复现", section 2.3). */
typedef struct gpt2_config {
    int32_t vocab;       /* V >= 1 */
    int32_t block_size;  /* maximum sequence length, rows of the position table */
    int32_t n_embd;      /* C; must be a multiple of n_head */
    int32_t n_head;      /* H; head size d = C / H */
    int32_t n_layer;     /* L >= 1 */
    int32_t mlp_hidden;  /* F (4C on the pages) */
    int32_t bias;        /* 1: Linear layers carry biases (LM head never does) */
    int32_t dtype;       /* GPT2_DTYPE_* */
    float ln_eps;        /* LayerNorm epsilon (1e-5, the nn.LayerNorm default) */
    /* The minigpt page's literal model (its section 二, minigpt.py) differs from the
     * GPT-2 readings in two switches; both 0 is GPT-2:
     * gelu_erf    1: the MLP activation is nn.GELU()'s exact form u Phi(u)
     *                (0: the tanh approximation the karpathy page's GELU section
     *                says GPT-2 uses);
     * untied_head 1: the LM head has a weight of its own, tensor "lm_head" [V, C]
     *                placed after lnf_b (minigpt's lm_head Linear, no bias); wte
     *                then gets only the embedding's gradient
     *                (0: the head reuses wte). Other values are GPT2_EINVAL. */
    int32_t gelu_erf;
    int32_t untied_head;
    /* Training-mode dropout probability p in [0, 1) (minigpt's cfg.dropout; 0:
     * none, the GPT-2 readings). With p > 0 a GPT2_MODE_TRAIN forward drops, as
     * minigpt.py's block does in model.train(): every head's attention weights
     * after the softmax, the attention projection's output and the FeedForward's
     * output, each element kept with probability 1 - round(65536 p) / 65536 and
     * scaled by 1 / (1 - p); the backward uses the same masks. The masks are
     * Philox4x32-10 draws under the key gpt2_set_dropout_seed sets (the element
     * numbering is documented there). EVAL and GENERATE contexts never drop. */
    float dropout;
} gpt2_config;

/* One named parameter tensor in the flat buffers. */
typedef struct gpt2_tensor_desc {
    char name[24];      /* "wte", "wpe", "h<l>.ln1_g", "h<l>.w_qkv", ..., "lnf_b" */
    int32_t layer;      /* block index, -1 for global tensors */
    int32_t decay;      /* 1 if AdamW decays it under GPT2_DECAY_MATRICES */
    int64_t offset;     /* element offset into params / grads / adam_m / adam_v */
    int64_t rows;       /* logical shape rows x cols, row-major, cols contiguous */
    int64_t cols;       /*   (vectors: rows = 1) */
    int64_t reserved;   /* elements reserved at offset (>= rows*cols; the rest stays 0) */
} gpt2_tensor_desc;

/* Caller-owned device memory. params/grads/adam_m/adam_v are fp32 arrays of the
 * n_flat elements gpt2_query_sizes reports, laid out per gpt2_param_table; padding
 * elements must be zero. The arena holds activations, low-precision weight copies
 * and scratch; its contents are private to the library. */
typedef struct gpt2_buffers {
    float* params;
    float* grads;
    float* adam_m;
    float* adam_v;
    void* arena;
    size_t arena_bytes;
} gpt2_buffers;

typedef struct gpt2_ctx gpt2_ctx;

/* ------------------------------------------------------------------ sizes and layout (host only) */
/* Flat length of the parameter buffers and arena bytes needed for batch B x T in
 * `mode`. T may be below block_size (positions 0..T-1 are used, minigpt page 3.7).
 * Returns GPT2_EINVAL for an invalid config, B < 1, T < 1 or T > block_size. */
int gpt2_query_sizes(const gpt2_config* cfg, int32_t B, int32_t T, int32_t mode,
                     size_t* n_flat, size_t* arena_bytes);

/* Exact parameter count (tied head counted once), or a negative code. */
int64_t gpt2_num_params(const gpt2_config* cfg);

/* Writes up to `cap` descriptors; returns the number of tensors (or a negative
 * code). Call with cap = 0 to size the array. */
int gpt2_param_table(const gpt2_config* cfg, gpt2_tensor_desc* out, int32_t cap);

/* Learning rate at iteration `it`: linear warmup to max_lr over `warmup`
 * iterations, cosine decay to min_lr at max_iters, min_lr after (the knobs of
 * train_gpt2.py, nanogpt page section 2.3; the curve's shape is a reading). */
double gpt2_lr_cosine(int64_t it, double max_lr, double min_lr, int64_t warmup, int64_t max_iters);

const char* gpt2_strerror(int code);

/* ------------------------------------------------------------------ the training step */
/* Validates, plans the arena for B x T, clears the status word and writes the
 * low-precision weight copies from bufs->params. hip_stream: a hipStream_t (NULL =
 * the null stream). On success *out owns a host-side plan; free with gpt2_destroy. */
int gpt2_init(gpt2_ctx** out, const gpt2_config* cfg, const gpt2_buffers* bufs, int32_t B, int32_t T,
              int32_t mode, void* hip_stream);

/* Re-derive the low-precision weight copies after the caller rewrote params
 * (loading a checkpoint, re-synchronising with another implementation). */
int gpt2_refresh_weights(gpt2_ctx* ctx);

/* Key of the dropout masks of the following TRAIN forwards (default 0); change
 * it every step for fresh masks. Element e of site s (0: attention weights, e =
 * ((b H + h) T + i) T + j for query i, key j of head h in sequence b; 1: the
 * projection output and 2: the FeedForward output, e = m C + c for row m = b T +
 * t) in layer l is kept when 16-bit half e % 8 (low half of word 0 first) of
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) at counter (e / 8 low and
 * high words, s, l) under key (seed low, seed high) is >= round(65536 p).
 * GPT2_ESTATE unless the context is a TRAIN context with p > 0. */
int gpt2_set_dropout_seed(gpt2_ctx* ctx, uint64_t seed);

/* Forward pass over d_idx [B*T] int32 (row-major [B][T]). With d_targets [B*T]
 * it also writes the mean cross-entropy over all B*T positions to *d_loss (one
 * float, device) and, in TRAIN mode, prepares the logits gradient for
 * gpt2_backward. d_argmax (nullable) receives each position's argmax over the
 * vocabulary (lowest index on ties). d_targets may be NULL for logits-only use
 * (then d_loss is ignored and backward is not possible). */
int gpt2_forward(gpt2_ctx* ctx, const int32_t* d_idx, const int32_t* d_targets, float* d_loss,
                 int32_t* d_argmax);

/* Backward of the last TRAIN forward. Gradients of loss_scale * mean loss are
 * written (zero_grads = 1, the optimizer.zero_grad of the minigpt loop) or added
 * (zero_grads = 0: gradient accumulation over micro-batches, loss_scale =
 * 1/accum_steps) into bufs->grads. */
int gpt2_backward(gpt2_ctx* ctx, float loss_scale, int32_t zero_grads);

#define GPT2_DECAY_ALL 0       /* every parameter decays (one param group, as minigpt's AdamW) */
#define GPT2_DECAY_MATRICES 1  /* only tensors with desc.decay = 1 (2-D weights and embeddings) */

/* Global L2 norm of the gradients (written to *d_grad_norm if non-NULL); if
 * clip > 0 and the norm exceeds it, gradients are scaled by clip/(norm + 1e-6).
 * Then one AdamW update (decoupled decay: p *= 1 - lr*wd, moments, bias
 * correction with step t >= 1, p -= lr * mhat / (sqrt(vhat) + eps)) over the
 * flat buffers, and the low-precision weight copies are refreshed. */
int gpt2_adamw_step(gpt2_ctx* ctx, float lr, float beta1, float beta2, float eps, float weight_decay,
                    int32_t t, float clip, int32_t decay_mode, float* d_grad_norm);

/* Autoregressive generation (MiniGPT.generate on the minigpt page, section 二 and
 * walkthrough 3.8) for a context made with GPT2_MODE_GENERATE (B sequences, T =
 * block_size). d_prompt: device int32 [B, T0], T0 >= 1. d_out: device int32
 * [B, T0 + n_new], receives the prompt followed by n_new drawn tokens. Each new
 * token: crop the sequence to its last block_size tokens, run the model, take
 * the last position's logits over `temperature` (> 0), softmax, and draw: the
 * token is the smallest k whose cumulative probability (index order) exceeds
 * u = d_uniform[b * n_new + i] (device fp32 [B, n_new], u in [0, 1); the pages
 * leave multinomial's procedure open, this is inverse-CDF sampling with the
 * caller's random numbers; u at or above the rounded total gives the last token
 * with nonzero probability). Keys and values of the window are cached; once the
 * sequence is longer than block_size the window slides and is recomputed from
 * its start each step. An id outside [0, V) sets GPT2_STATUS_TOKEN_RANGE.
 * Enqueue-only on the context's stream; GPT2_ESTATE for other modes. */
int gpt2_generate(gpt2_ctx* ctx, const int32_t* d_prompt, int32_t T0, int32_t n_new, float temperature,
                  const float* d_uniform, int32_t* d_out);

/* ------------------------------------------------------------------ character-level data
 * prepare_data and get_batch of minigpt.py (the minigpt page, section 二; walkthrough
 * 3.2). A character is one byte of the text (the same as the page's str for ASCII).
 *
 * gpt2_char_vocab: the sorted distinct bytes of text[0, n) into chars[256]; returns
 *   the vocabulary size (GPT2_EINVAL on null pointers). Host only.
 * gpt2_char_encode / gpt2_char_decode: ids[i] = position of text[i] in chars[0,
 *   vocab), and back; GPT2_EINVAL on a byte outside the vocabulary or an id outside
 *   [0, vocab). Host only.
 * gpt2_split_point: int(ratio * n), the end of the training split (ratio in [0, 1]).
 * gpt2_batch_windows: device int32 token stream d_data[0, n), device int64 window
 *   starts d_offsets[B] (get_batch draws them from [0, n - T - 1); the caller
 *   supplies them) -> device int32 d_x[B, T] = d_data[off_b + t], d_y[B, T] =
 *   d_data[off_b + t + 1]. A start outside [0, n - T - 1] zeroes its rows and sets
 *   GPT2_STATUS_WINDOW_RANGE in *d_status (device uint32, nullable). Enqueued on
 *   hip_stream; the caller owns every buffer. */
int32_t gpt2_char_vocab(const uint8_t* text, int64_t n, uint8_t* chars);
int gpt2_char_encode(const uint8_t* text, int64_t n, const uint8_t* chars, int32_t vocab, int32_t* ids);
int gpt2_char_decode(const int32_t* ids, int64_t n, const uint8_t* chars, int32_t vocab, uint8_t* text);
int64_t gpt2_split_point(int64_t n, double ratio);
int gpt2_batch_windows(const int32_t* d_data, int64_t n, const int64_t* d_offsets, int32_t B, int32_t T,
                       int32_t* d_x, int32_t* d_y, uint32_t* d_status, void* hip_stream);

/* Synchronises the stream and reads the sticky status word into *bits (nullable).
 * Returns GPT2_EDEVICE if any bit is set, else GPT2_OK. gpt2_clear_status resets it. */
int gpt2_sync_status(gpt2_ctx* ctx, uint32_t* bits);
int gpt2_clear_status(gpt2_ctx* ctx);

/* Per-launch timing for profiling. After gpt2_timing_begin(ctx, prefix), every
 * kernel launch of the step whose label starts with `prefix` is bracketed by HIP
 * events recorded on the step's stream. gpt2_timing_end synchronises the stream,
 * returns the summed event-measured duration (ms) and the number of launches
 * timed, and stops timing. Labels: "embed.fwd", "ln.fwd", "gemm.fwd.{qkv,proj,
 * fc,fc2,head}", "attn.fwd", "ce", "loss", "gemm.dgrad.{head,fc2,fc,proj,qkv}",
 * "gemm.wgrad.{head,fc2,fc,proj,qkv}", "ln.bwd", "colsum", "bias",
 * "attn.bwd.{dq,dkdv}" (bf16, head size 64; "attn.bwd" otherwise), "embed.bwd",
 * "gradnorm", "adamw", "dropout.mask" (with dropout; on the second stream when
 * there is one, so its events overlap the forward's). A prefix also times the labels that extend it by a
 * '.'-separated part ("attn.bwd" covers both backward launches); an empty
 * prefix times every launch. */
int gpt2_timing_begin(gpt2_ctx* ctx, const char* prefix);
int gpt2_timing_end(gpt2_ctx* ctx, float* total_ms, int32_t* launches);

/* Byte offset inside the arena of an activation, for inspection by tests:
 * name in {"x", "xmid", "ln1", "ln2", "qkv", "att", "lse", "fch", "fcg", "xf",
 * "logits", "loss_rows"}; layer ignored for the last three. *elem_bytes receives
 * 2 or 4. In TRAIN mode "logits" holds the logits gradient after a forward with
 * targets. "fcg" is the GELU output of the MLP's first layer and "fch" the GELU
 * derivative at its pre-activation (the factor the backward applies). With
 * dropout, "drop_attn" (rows B H T, cols ceil(T / 64)), "drop_proj" and
 * "drop_fc2" (ceil(B T C / 64) rows, 1 col) are the layer's keep bits of the last
 * TRAIN forward as 8-byte words, bit k of word w the element numbered as in
 * gpt2_set_dropout_seed (attention: key 64 w' + k of row (b H + h) T + i, w' the
 * column; residual sites: element 64 w + k); attention bits past the diagonal
 * are zero. */
int gpt2_arena_tensor(const gpt2_ctx* ctx, const char* name, int32_t layer, size_t* byte_offset,
                      int32_t* elem_bytes, int64_t* rows, int64_t* cols);

void gpt2_destroy(gpt2_ctx* ctx);

/* ------------------------------------------------------------------ single operations
 * The kernels of the step, callable one at a time on caller device buffers (for
 * kernel-level tests and profiling). dtype selects fp32 or bf16 activations as in
 * gpt2_config.dtype; "act" buffers below are float* (F32) or bf16 bit patterns
 * (uint16_t*, BF16). All matrices are row-major with the stated shapes. */

/* Y[M,N] = X[M,K] . W[N,K]^T (+ bias[N]) (nn.Linear, minigpt page section 二).
 * X, W, Y: act; bias: fp32 or NULL. */
int gpt2_op_linear_fwd(int32_t dtype, int64_t M, int32_t N, int32_t K, const void* d_X, const void* d_W,
                       const float* d_bias, void* d_Y, void* hip_stream);
/* dX[M,K] = dY[M,N] . W (act, overwritten; nullable); dW[N,K] (fp32) = or += dY^T X;
 * db[N] (fp32, nullable) = or += column sums of dY. accumulate: 0 overwrite, 1 add. */
int gpt2_op_linear_bwd(int32_t dtype, int64_t M, int32_t N, int32_t K, const void* d_dY, const void* d_X,
                       const void* d_W, void* d_dX, float* d_dW, float* d_db, int32_t accumulate,
                       void* hip_stream);
/* y (act) = LayerNorm(x fp32 [rows, C]) with g, b fp32; mean, rstd fp32 [rows]. */
int gpt2_op_layernorm_fwd(int32_t dtype, int64_t rows, int32_t C, const float* d_x, const float* d_g,
                          const float* d_b, float eps, void* d_y, float* d_mean, float* d_rstd, void* hip_stream);
/* dx (fp32) += LayerNorm backward of dy (fp32); dg, db (fp32 [C]) overwritten. */
int gpt2_op_layernorm_bwd(int64_t rows, int32_t C, const float* d_dy, const float* d_x, const float* d_mean,
                          const float* d_rstd, const float* d_g, float* d_dx, float* d_dg, float* d_db,
                          void* hip_stream);
/* Causal multi-head attention over qkv (act [B*T, 3C]) -> out (act [B*T, C]),
 * lse (fp32 [B, H, T], the log-sum-exp of each scaled score row). */
int gpt2_op_attention_fwd(int32_t dtype, int32_t B, int32_t T, int32_t C, int32_t H, const void* d_qkv,
                          void* d_out, float* d_lse, void* hip_stream);
/* dqkv (act [B*T, 3C], overwritten) from dout (act [B*T, C]) and the forward's
 * qkv, out and lse. */
int gpt2_op_attention_bwd(int32_t dtype, int32_t B, int32_t T, int32_t C, int32_t H, const void* d_qkv,
                          const void* d_out, const float* d_lse, const void* d_dout, void* d_dqkv,
                          void* hip_stream);
/* Row-wise cross-entropy over logits (act [rows, ld], first V columns valid):
 * loss_rows (fp32 [rows]) = lse - z[target]; if write_grad, logits are
 * overwritten with softmax - onehot (columns >= V set to 0); argmax (nullable). */
int gpt2_op_cross_entropy(int32_t dtype, int64_t rows, int32_t V, int32_t ld, void* d_logits,
                          const int32_t* d_targets, float* d_loss_rows, int32_t* d_argmax, int32_t write_grad,
                          void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_MI355X_H */
