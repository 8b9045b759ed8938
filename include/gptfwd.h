/*
 * gptfwd.h -- C ABI of libgptfwd: the nanochat GPT forward pass with next-token loss on AMD
 * MI355X (gfx950).
 *
 * The operation (sources cited by page title and section):
 *   "The Mathematics of Karpathy's nanochat", sections "High-Level Forward Pass" and
 *   "Pseudocode: One Training Step": x = RMSNorm(W_E[t]); x0 = x; for every layer l:
 *   x = lambda_l x + mu_l x0; x += W_O Attn(RoPE + QK-norm of W_Q/W_K/W_V RMSNorm(x));
 *   x += W_2 relu(W_1 RMSNorm(x))^2; then zhat = cap tanh(W_U RMSNorm(x) / cap) and the
 *   cross-entropy of zhat against the next token ("Logit Softcap", "Cross-Entropy Loss").
 *   Attention is causal with a per-layer window w_l: query i sees key j iff j <= i and
 *   i - j < w_l ("Scaled Dot-Product Attention with Sliding Window"); the short/long window
 *   pattern is tiled over the layers with the last layer always long ("nanochat depth sweep",
 *   section "Architecture").  The logit of a visible pair is attn_scale * <q_hat, k_hat>.
 *   Input/target shift: "Reading nanochat Source: From Configuration to a Training Step",
 *   section 2 -- targets[b][t] is the token that follows tokens[b][t].
 *
 * Conventions
 *   - All array pointers are DEVICE pointers unless marked "host".  All matrices are row-major;
 *     weights are [out_features, in_features].
 *   - Ownership: the caller owns every buffer (weights, inputs, outputs, workspace).  The
 *     library allocates no memory and keeps no pointer after the enqueued work completes.  It
 *     keeps no state: calls with distinct workspaces may run concurrently on different streams.
 *   - Asynchrony: gpt_fwd_loss only enqueues work on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns; results are valid once the stream reaches that point.
 *   - Errors: every argument error detectable on the host is reported before any work is
 *     enqueued, and no output is touched.  A failed kernel launch returns GPT_E_HIP.  Invalid
 *     token or target ids are detected on the device: the affected per-token losses are NaN and
 *     gpt_device_status() reports GPT_E_DEVICE_INPUT.
 *   - Precision: with GPT_BF16 the weights and the GEMM/attention operands are bf16; products
 *     accumulate in fp32, and the residual stream, every normalisation statistic, the softmax
 *     and the logits are fp32.  With GPT_F32 everything is fp32.
 */
#ifndef GPTFWD_H
#define GPTFWD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT_OK = 0,
  GPT_E_INVALID_ARG = -1,  /* NULL pointer, non-positive size, inconsistent shape */
  GPT_E_UNSUPPORTED = -2,  /* valid model, but outside what the kernels implement (see gpt_cfg) */
  GPT_E_WORKSPACE = -3,    /* workspace NULL, too small or not 256-byte aligned */
  GPT_E_HIP = -4,          /* a HIP call or kernel launch failed */
  GPT_E_DEVICE_INPUT = -5  /* (gpt_device_status) a token or target id was out of range */
} gpt_status;

typedef enum { GPT_F32 = 0, GPT_BF16 = 1 } gpt_dtype;

/* Model and batch shape.  Supported: head_dim in {64, 128}; n_head % n_kv_head == 0;
 * d_model, n_head*head_dim and mlp_dim multiples of 64; vocab >= 2; for GPT_BF16 seq_len a
 * multiple of 64 and n_kv_head*head_dim a multiple of 128.  d_model <= 8192.  batch >= 1 and
 * seq_len >= 1: an empty batch is GPT_E_INVALID_ARG, not a call that does nothing.  32-bit
 * limits (GPT_E_UNSUPPORTED beyond them): batch*seq_len <= 2^30, vocab*d_model <= 2^31,
 * seq_len*head_dim/2 < 2^31, and for GPT_BF16 one sequence's q/k rows,
 * seq_len*(n_head+n_kv_head)*head_dim*2 bytes, at most 2^31 - 1. */
typedef struct {
  int32_t n_layer;      /* L */
  int32_t d_model;      /* C, residual width */
  int32_t n_head;       /* H, query heads */
  int32_t n_kv_head;    /* Hkv, key/value heads; query head h reads KV head h*Hkv/H */
  int32_t head_dim;     /* D */
  int32_t mlp_dim;      /* F, MLP hidden width (4C in nanochat) */
  int32_t vocab;        /* V */
  int32_t seq_len;      /* T, tokens per packed row */
  int32_t batch;        /* B, rows */
  const int32_t *window;/* host [n_layer]: keys visible to a query, itself included, >= 1;
                           a value >= seq_len means full causal attention */
  float softcap;        /* cap > 0 of zhat = cap * tanh(z / cap); nanochat uses 15 */
  float rope_base;      /* RoPE theta; nanochat uses 100000 */
  float attn_scale;     /* logit scale applied to <q_hat, k_hat>, e.g. 1/sqrt(head_dim) */
  float norm_eps;       /* eps inside every RMSNorm's square root, >= 0 (1e-6) */
  int32_t dtype;        /* gpt_dtype of weights and activations */
  const uint8_t *has_ve;/* host [n_layer] or NULL: nonzero where the layer mixes a value
                           embedding into v ("Value Embeddings (ResFormer)": the pages select
                           l % 2 == (n_layer - 1) % 2); needs d_model >= 12, and head_dim 128
                           for GPT_BF16 */
  int32_t looped;       /* 0, or 1 for the two-pass looped trunk ("looped-nanochat-d24", section
                           "What is the routing loop?"): pass p in {0, 1} starts from
                           RMSNorm(W_E[t] + pass_emb[p]); pass-2 layer l adds
                           softplus(gate_logit[l]) * attn_scale * <q1, k1> of pass-1 layer l to
                           its logits; the loss comes from pass 2.  GPT_BF16 needs head_dim 128. */
  int32_t nested_c1;    /* 0, or the width c1 of the inner block of a two-block nested model
                           (StairFormer, "Fully Nested Transformers", opening section and
                           "Reproducing the main experiment"): every per-layer linear is block
                           lower triangular, every RMSNorm on the residual stream a PrefixRMSNorm
                           (columns [0, c1) normed by their own RMS, the rest by the whole row's),
                           so columns [0, c1) of the stream evolve as a standalone model of width
                           c1 would.  Every partitioned dimension splits in the proportion
                           c1 : d_model: the inner block holds the first H1 = n_head*c1/d_model
                           query heads, Hkv1 = n_kv_head*c1/d_model KV heads and F1 =
                           mlp_dim*c1/d_model hidden units.  Needs 0 < c1 <= d_model, c1 and F1
                           multiples of 64, exact splits, no value embeddings and looped = 0; for
                           GPT_BF16 also H1*head_dim and Hkv1*head_dim multiples of 128. */
} gpt_cfg;

/* Weights: borrowed device memory of type cfg->dtype (float or bf16), row-major [out, in].
 * Per-layer matrices are given as HOST arrays of n_layer device pointers.  Every device
 * pointer must be 16-byte aligned.
 *
 * Nested models (cfg->nested_c1 > 0) store only the live blocks of each block lower triangular
 * linear [out, in] with inner shares out1, in1 ("Fully Nested Transformers", section "What's
 * here": only live weights are stored): row block 1 [out1, in1] row-major, immediately
 * followed by row block 2 [out - out1, in] row-major.  (out1, in1) is (H1*D, c1) for wq,
 * (Hkv1*D, c1) for wk and wv, (c1, H1*D) for wo, (F1, c1) for w1 and (c1, F1) for w2.  wte and
 * lm_head stay dense [vocab, d_model]; the inner model reads their first c1 columns. */
typedef struct {
  const void *wte;            /* [vocab, d_model] token embedding W_E */
  const void *lm_head;        /* [vocab, d_model] unembedding W_U (untied) */
  const float *resid_lambda;  /* device fp32 [n_layer]: lambda_l */
  const float *x0_lambda;     /* device fp32 [n_layer]: mu_l */
  const void *const *wq;      /* host [n_layer] -> [n_head*head_dim, d_model] */
  const void *const *wk;      /* host [n_layer] -> [n_kv_head*head_dim, d_model] */
  const void *const *wv;      /* host [n_layer] -> [n_kv_head*head_dim, d_model] */
  const void *const *wo;      /* host [n_layer] -> [d_model, n_head*head_dim] */
  const void *const *w1;      /* host [n_layer] -> [mlp_dim, d_model] */
  const void *const *w2;      /* host [n_layer] -> [d_model, mlp_dim] */
  /* Value embeddings, read only on layers with cfg->has_ve[l] (the arrays may be NULL when
   * cfg->has_ve is NULL; entries of other layers are ignored):
   *   ve[l]      [vocab, n_kv_head*head_dim] table; row t is added to token t's v heads
   *   ve_gate[l] [n_kv_head, 12] gate weights: g = 3 sigmoid(x_tilde[:12] . ve_gate[l][h])
   *              per KV head h, x_tilde the normalised input of the layer's projections */
  const void *const *ve;      /* host [n_layer] */
  const void *const *ve_gate; /* host [n_layer] */
  /* Looped trunk only (cfg->looped): */
  const void *pass_emb;       /* [2, d_model] per-pass embeddings */
  const float *gate_logit;    /* device fp32 [n_layer] routing gate logits */
} gpt_weights;

/* Validate a configuration without touching any device.  Returns GPT_OK, GPT_E_INVALID_ARG or
 * GPT_E_UNSUPPORTED. */
gpt_status gpt_validate(const gpt_cfg *cfg);

/* Bytes of device workspace gpt_fwd_loss needs for this configuration (0 if the configuration
 * does not validate). */
size_t gpt_workspace_bytes(const gpt_cfg *cfg);

/* Forward pass plus next-token loss over tokens [batch, seq_len].
 *   tokens     device int32 [B, T], ids in [0, vocab)
 *   targets    device int32 [B, T], ids in [0, vocab) or -1 (ignored position); may be NULL, in
 *              which case no loss is computed and `logits` must be non-NULL
 *   loss       device fp32 [B, T] out: per-token loss, 0 at ignored positions; required iff
 *              targets is non-NULL
 *   mean_loss  device fp32 [1] out: mean over positions with target != -1 (NaN if none);
 *              required iff targets is non-NULL
 *   logits     device fp32 [B, T, vocab] out: softcapped logits zhat, or NULL (the default
 *              path never materialises the logits)
 *   workspace  device scratch of at least gpt_workspace_bytes(cfg), 256-byte aligned; its
 *              contents on entry do not matter
 * Returns GPT_OK once everything is enqueued on `stream` (hipStream_t). */
gpt_status gpt_fwd_loss(const gpt_cfg *cfg, const gpt_weights *w, const int32_t *tokens,
                        const int32_t *targets, float *loss, float *mean_loss, float *logits,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Measurement hook.  Kinds of launch in the forward pass, one per layer unless noted:
 * GPT_KERNEL_QKV          q/k/v projection with its RoPE + QK-norm epilogue (bf16: one or two
 *                         GEMM kernels)
 * GPT_KERNEL_ATTENTION    windowed causal attention
 * GPT_KERNEL_ATTN_OUT     attention output projection + residual add
 * GPT_KERNEL_MLP_UP       MLP up-projection with the ReLU^2 epilogue
 * GPT_KERNEL_MLP_DOWN     MLP down-projection + residual add (+ the next layer's x0 mix)
 * GPT_KERNEL_LM_HEAD      lm_head GEMM with the softcapped cross-entropy epilogue (once)
 * The fp32 path times only GPT_KERNEL_LM_HEAD. */
typedef enum {
  GPT_KERNEL_QKV = 1,
  GPT_KERNEL_ATTENTION = 2,
  GPT_KERNEL_ATTN_OUT = 3,
  GPT_KERNEL_MLP_UP = 4,
  GPT_KERNEL_MLP_DOWN = 5,
  GPT_KERNEL_LM_HEAD = 6
} gpt_kernel_kind;

/* Caller-owned timing record: begin[i] and end[i] are HIP events (hipEvent_t, created by the
 * caller with timing enabled) that take the start time of the first kernel and the end time of
 * the last kernel of the i-th launch of `kind` (in launch order, while i < capacity), stamped
 * by the dispatches themselves (hipExtLaunchKernelGGL).  `recorded` (out) counts the pairs
 * used by the call.  The library keeps no pointer to the record after returning. */
typedef struct {
  int32_t kind;          /* gpt_kernel_kind */
  int32_t capacity;      /* pairs available in begin/end (>= 0) */
  void *const *begin;    /* host [capacity] hipEvent_t */
  void *const *end;      /* host [capacity] hipEvent_t */
  int32_t recorded;      /* out */
} gpt_launch_timing;

/* gpt_fwd_loss, plus kernel timestamps for the launches that `timing` selects (NULL: exactly
 * gpt_fwd_loss).  Meant for measurement runs: the timed launches take a different (slower to
 * enqueue) host path.  GPT_E_INVALID_ARG for an unknown kind, a negative capacity or NULL event
 * arrays with capacity > 0. */
gpt_status gpt_fwd_loss_timed(const gpt_cfg *cfg, const gpt_weights *w, const int32_t *tokens,
                              const int32_t *targets, float *loss, float *mean_loss,
                              float *logits, void *workspace, size_t workspace_bytes,
                              void *stream, gpt_launch_timing *timing);

/* Nested models: the full model's outputs (as gpt_fwd_loss) and, from the same single pass,
 * those of the inner model -- the kfront=1 submodel of "Fully Nested Transformers", section
 * "Reproducing the main experiment": the cross-entropy of cap * tanh(z1 / cap) with z1 the
 * first c1 columns of the final PrefixRMSNorm'd stream against the first c1 columns of
 * lm_head.  loss_k1 [B, T], mean_k1 [1] and logits_k1 [B, T, vocab] follow the rules of loss,
 * mean_loss and logits; the k1 outputs may all be NULL (then this is gpt_fwd_loss_timed).
 * GPT_E_INVALID_ARG if cfg->nested_c1 == 0.  `timing` as in gpt_fwd_loss_timed (NULL: none);
 * the inner and outer row-block launches of one step share a pair, and the two lm_head passes
 * take one pair each (full model first). */
gpt_status gpt_fwd_loss_nested(const gpt_cfg *cfg, const gpt_weights *w, const int32_t *tokens,
                               const int32_t *targets, float *loss, float *mean_loss,
                               float *logits, float *loss_k1, float *mean_k1, float *logits_k1,
                               void *workspace, size_t workspace_bytes, void *stream,
                               gpt_launch_timing *timing);

/* ---- Decoding ("The Mathematics of Karpathy's nanochat", section "Inference: Generating
 * Text": an autoregressive loop that takes the logits at the last position and samples the
 * next token).  gpt_decode_step runs the forward pass for ONE new token per row at position
 * pos[b], reading the keys and values of positions < pos[b] from a KV cache that earlier steps
 * of the same row filled and writing those of pos[b] into it; its logits are those the full
 * forward gives at position pos[b] of the sequence so far (attention is causal).  Here
 * cfg->batch is the number of rows (1..32) and cfg->seq_len the cache capacity T (<= 8192;
 * at most 8 query heads per KV head; with GPT_BF16, d_model <= 4096);
 * the per-layer windows apply as in the forward.  Base models only: no value embeddings,
 * looped trunk or nested model (GPT_E_UNSUPPORTED).
 *
 * KV cache layout (device, cfg->dtype, caller-owned, contents before a row's first step do not
 * matter): for layer l, k_hat at [l][0][b][g][t][d] and v at [l][1][b][g][t][d], dimensions
 * [n_layer][2][batch][n_kv_head][seq_len][head_dim]; k_hat is the RoPE'd, normalised key. */
size_t gpt_kv_cache_bytes(const gpt_cfg *cfg);         /* 0 if cfg does not validate for decoding */
size_t gpt_decode_workspace_bytes(const gpt_cfg *cfg); /* 0 likewise */

/*   tokens     device int32 [B]: the token at position pos[b] of row b, in [0, vocab)
 *   pos        device int32 [B]: its position, in [0, seq_len)
 *   kv_cache   device, gpt_kv_cache_bytes(cfg), 256-byte aligned
 *   logits     device fp32 [B, vocab] out: softcapped logits zhat at pos[b]
 *   workspace  device, gpt_decode_workspace_bytes(cfg), 256-byte aligned (contents on entry do
 *              not matter)
 * Enqueues only (no host synchronisation, no allocation), so a step can be captured in a HIP
 * graph and replayed with new tokens/pos values.  A row whose token or position is out of range
 * gets NaN logits, writes nothing into the cache, and gpt_device_status(workspace) reports
 * GPT_E_DEVICE_INPUT. */
gpt_status gpt_decode_step(const gpt_cfg *cfg, const gpt_weights *w, const int32_t *tokens,
                           const int32_t *pos, void *kv_cache, float *logits, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Prefill: fill the KV cache from ONE forward pass over a prompt batch tokens [B, prompt_len]
 * (device int32, prompt_len <= seq_len; GPT_BF16 needs prompt_len % 64 == 0, as the forward
 * does) instead of prompt_len decode steps, and return in logits [B, vocab] (device fp32) the
 * softcapped logits at each row's last prompt position, len_b - 1, with len_b = lens[b] (device
 * int32 [B], 1 <= len_b <= prompt_len; NULL: every row has prompt_len tokens).  Positions
 * [0, prompt_len) of every row are written to the cache; decoding a row continues at pos =
 * len_b, whose steps overwrite the padded positions before any query can see them, so ragged
 * prompts share one padded batch.  A row with an invalid length gets NaN logits and raises the
 * device input flag.  The workspace is gpt_prefill_workspace_bytes(cfg) (the forward's). */
size_t gpt_prefill_workspace_bytes(const gpt_cfg *cfg); /* 0 if cfg does not validate for decoding */
gpt_status gpt_prefill(const gpt_cfg *cfg, const gpt_weights *w, const int32_t *tokens,
                       int32_t prompt_len, const int32_t *lens, void *kv_cache, float *logits,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Sampling controls of the same section: for each row b of logits [batch, vocab] (device fp32),
 * out[b] (device int32) = the first index of the largest logit if temperature == 0; otherwise
 * the tokens whose logit is >= the top_k-th largest are kept (ties at the threshold stay;
 * top_k <= 0 or >= vocab keeps all), p_v = exp((z_v - max z) / temperature) over them, and
 * out[b] is the first token in vocabulary order whose running sum of p exceeds u[b] * sum p
 * (u device fp32 [batch], uniform draws in [0, 1) supplied by the caller: the library draws no
 * random numbers).  GPT_E_INVALID_ARG for a negative or non-finite temperature, batch < 1 or
 * vocab < 1, or NULL pointers. */
gpt_status gpt_sample(const float *logits, int32_t batch, int32_t vocab, int32_t top_k,
                      float temperature, const float *u, int32_t *out, void *stream);

/* Synchronise `stream`, then report whether any gpt_fwd_loss (or gpt_decode_step) call that
 * used this workspace saw an out-of-range token, target id or position since the workspace's
 * last call began (GPT_OK or GPT_E_DEVICE_INPUT; GPT_E_HIP if synchronising failed). */
gpt_status gpt_device_status(void *workspace, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gpt_fwd_loss with the workspace taken from a fixed
 * array inside this library instead of an argument.  The array holds GPT_NOALLOC_MAX_BYTES
 * (64 MiB) on every GPU the library runs on, from the first such call on that GPU until the
 * process ends; configurations whose gpt_workspace_bytes() exceeds it are refused with
 * GPT_E_WORKSPACE before any HIP call (a configuration that does not validate returns
 * gpt_validate()'s status), and nothing is allocated, by this call or the forward pass.  The
 * other arguments, their checks and the results are those of gpt_fwd_loss.  Every call on one
 * GPU uses that GPU's single array, which keeps the last call's contents: calls that overlap on
 * one GPU (different streams, or host threads) race, and must be ordered by the caller.  The
 * array's device error flags are not readable through gpt_device_status(): out-of-range ids
 * still show as NaN per-token losses. */
#define GPT_NOALLOC_MAX_BYTES (64u << 20)
gpt_status gpt_fwd_loss_noalloc(const gpt_cfg *cfg, const gpt_weights *w, const int32_t *tokens,
                                const int32_t *targets, float *loss, float *mean_loss,
                                float *logits, void *stream);

/* Static description of a status code (never NULL). */
const char *gpt_status_string(gpt_status s);

#ifdef __cplusplus
}
#endif

#endif /* GPTFWD_H */
