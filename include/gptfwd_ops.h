/*
 * gptfwd_ops.h -- component entry points of libgptfwd.
 *
 * Each call enqueues exactly the kernel(s) that gpt_fwd_loss uses for one step of the forward
 * pass, on caller-owned device buffers, so every step can be checked and timed on its own.
 * Conventions (ownership, asynchrony on `stream`, status codes, row-major layouts, device
 * pointers unless marked host) are those of gptfwd.h.  `dtype` is a gpt_dtype: GPT_BF16
 * activations/weights are bf16, GPT_F32 ones fp32; residual-stream buffers (x, x0) are always
 * fp32.  Host-detectable argument errors return before anything is enqueued.
 */
#ifndef GPTFWD_OPS_H
#define GPTFWD_OPS_H

#include "gptfwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Embedding + RMSNorm ("The Mathematics of Karpathy's nanochat", "High-Level Forward Pass"
 * steps 1-2, "RMS Normalization") fused with layer 0's mix and pre-attention norm:
 *   x0 = RMSNorm(wte[tokens]);  x = lam[0] x0 + mu[0] x0;  xn = RMSNorm(x).
 * tokens int32 [M]; wte [V, C]; lam, mu fp32 [>=1]; x0, x fp32 [M, C] out; xn [M, C] out.
 * flags: device uint32, bit 0 set when a token id is outside [0, V). C % 4 == 0, C <= 8192. */
gpt_status gpt_op_embed_norm(int32_t dtype, const int32_t *tokens, const void *wte,
                             const float *lam, const float *mu, float *x0, float *x, void *xn,
                             int32_t M, int32_t C, int32_t V, float eps, uint32_t *flags,
                             void *stream);

/* Residual mix and RMSNorm ("Residual Stream with Learnable Scalars"):
 *   if mix: x = lam[layer] x + mu[layer] x0 (in place);  xn = RMSNorm(x).
 * x fp32 [M, C] in/out; x0 fp32 [M, C] (unused without mix); xn [M, C] out. */
gpt_status gpt_op_mix_norm(int32_t dtype, float *x, const float *x0, const float *lam,
                           const float *mu, int32_t layer, int32_t mix, void *xn, int32_t M,
                           int32_t C, float eps, void *stream);

/* RoPE table ("Rotary Position Embeddings (RoPE)", Frequency Construction):
 * cs fp32 [T, D/2, 2] out with (cos, sin) of t * base^(-2j/D), evaluated in fp64.
 * GPT_E_UNSUPPORTED when T * D/2 does not fit a 32-bit index. */
gpt_status gpt_op_rope_table(float *cs, int32_t T, int32_t D, float base, void *stream);

/* RoPE then per-head RMSNorm, in place ("Rotary Position Embeddings (RoPE)", Rotation
 * Application; "QK-Norm with Sharpening" without the 1.15 gain): for every row r of qk
 * [M, ld] and head hh < nheads, the D values at column hh*D are rotated by the half-split rule
 * at position r % T and divided by their RMS.  cs from gpt_op_rope_table. D even, <= 128. */
gpt_status gpt_op_qk_rope_norm(int32_t dtype, void *qk, int32_t ld, const float *cs, int32_t M,
                               int32_t T, int32_t nheads, int32_t D, float eps, void *stream);

/* Linear layer out = a w^T ("Causal Self-Attention" projections, "Output Projection",
 * "Feed-Forward Network (MLP)"): a [M, K], w [N, K].  epi 0: out [M, N] = result (dtype);
 * epi 1: out [M, N] = max(0, result)^2 (dtype); epi 2: out fp32 [M, N] += result.
 * K % 64 == 0 for GPT_BF16. */
gpt_status gpt_op_linear(int32_t dtype, int32_t epi, const void *a, const void *w, int32_t M,
                         int32_t N, int32_t K, void *out, void *stream);

/* QKV projection as the forward pass runs it (GPT_BF16 only): [q|k|v] = xn [wq;wk;wv]^T with
 * xn [B*T, C]; q and k go to qk [B*T, (H+Hkv)*D] row-major, v to vt [B, Hkv, D, T].  If cs (a
 * table from gpt_op_rope_table) is non-NULL, every q and k head is rotated and RMS-normalised
 * (eps inside the root) in fp32 before rounding, exactly as gpt_op_qk_rope_norm would do to the
 * unrounded projection; this fused form needs T % 32 == 0 (else GPT_E_UNSUPPORTED).  C % 64 == 0, T % 4 == 0 and (H*D) % 128 == (Hkv*D) % 128 == 0 always. */
gpt_status gpt_op_qkv(const void *xn, const void *wq, const void *wk, const void *wv, int32_t B,
                      int32_t T, int32_t C, int32_t H, int32_t Hkv, int32_t D, const float *cs,
                      float eps, void *qk, void *vt, void *stream);

/* Windowed causal attention ("Scaled Dot-Product Attention with Sliding Window") on already
 * rotated and normalised q, k.  GPT_BF16: q/k from qk [B*T, (H+Hkv)*D], v from vt
 * [B, Hkv, D, T]; GPT_F32: q/k/v from qk [B*T, (H+2*Hkv)*D] and vt ignored.  o [B*T, H*D] out.
 * Query head h reads KV head h*Hkv/H.  D in {64, 128}.  GPT_BF16 also needs T % 64 == 0 and one
 * sequence's q/k rows under 2^31 bytes (T * (H+Hkv) * D * 2), else GPT_E_UNSUPPORTED. */
gpt_status gpt_op_attention(int32_t dtype, const void *qk, const void *vt, void *o, int32_t B,
                            int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t window,
                            float scale, void *stream);

/* Fused lm_head + softcap + cross-entropy ("Logit Softcap", "Cross-Entropy Loss"):
 * xf [M, C] (final-normed), wu [V, C]; targets int32 [M] (-1 = ignore) or NULL; tokens int32
 * [M] (only checked for range) ; loss fp32 [M] out; mean fp32 [1] out; logits fp32 [M, V] out
 * or NULL.  workspace: at least gpt_op_lm_head_ce_workspace(dtype, M, V) bytes, 256-aligned. */
size_t gpt_op_lm_head_ce_workspace(int32_t dtype, int32_t M, int32_t V);
gpt_status gpt_op_lm_head_ce(int32_t dtype, const void *xf, const void *wu, const int32_t *targets,
                             const int32_t *tokens, int32_t M, int32_t C, int32_t V, float cap,
                             float *loss, float *mean, float *logits, void *workspace,
                             size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTFWD_OPS_H */
