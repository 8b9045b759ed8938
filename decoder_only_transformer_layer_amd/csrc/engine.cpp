// libgptfwd host engine: argument validation, workspace planning and the launch sequence of
// the forward pass, behind the C ABI of include/gptfwd.h and include/gptfwd_ops.h.
//
// Layer order follows "The Mathematics of Karpathy's nanochat", sections "High-Level Forward
// Pass" and "Pseudocode: One Training Step"; see the header for the full statement.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "gptfwd.h"
#include "gptfwd_ops.h"
#include "kernels.h"

namespace {

using namespace gptk;

constexpr size_t ALIGN = 256;
inline size_t up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Layout {
  size_t flags, x, x0, xn, qk, vt, o, h, cs, ssp, partial, tgt, qk1, last, partial1, tgt1, total;
  int nnb;
};

// Prefill (gpt_prefill): the forward's layers also fill the decode cache (capacity T rows per
// (row, KV head)); the outputs are the logits at each row's last prompt position.
struct Prefill {
  void* cache;
  int T;
  const int32_t* lens;
  float* logits;
};

constexpr int VE_GATE_CH = 12;  // input channels of the value-embedding gate

bool any_ve(const gpt_cfg* c) {
  if (!c->has_ve) return false;
  for (int l = 0; l < c->n_layer; ++l)
    if (c->has_ve[l]) return true;
  return false;
}

// 32-bit index limits shared by the model and the per-step entry points: the RoPE table's entry
// index (T * D/2), and one sequence's q/k rows in the bf16 attention, which its K tiles read
// through a buffer resource of fewer than 2^31 bytes.
bool rope_fits(long T, long D) { return T * (D / 2) <= INT32_MAX - 255; }
bool attn_bf16_fits(long T, long H, long Hkv, long D) { return T * (H + Hkv) * D * 2 <= INT32_MAX; }

gpt_status validate(const gpt_cfg* c) {
  if (!c) return GPT_E_INVALID_ARG;
  if (c->n_layer < 1 || c->d_model < 1 || c->n_head < 1 || c->n_kv_head < 1 || c->head_dim < 1 ||
      c->mlp_dim < 1 || c->vocab < 2 || c->seq_len < 1 || c->batch < 1)
    return GPT_E_INVALID_ARG;
  if (c->n_head % c->n_kv_head) return GPT_E_INVALID_ARG;
  if (c->dtype != GPT_F32 && c->dtype != GPT_BF16) return GPT_E_INVALID_ARG;
  if (!c->window) return GPT_E_INVALID_ARG;
  for (int l = 0; l < c->n_layer; ++l)
    if (c->window[l] < 1) return GPT_E_INVALID_ARG;
  if (!(c->softcap > 0.f) || !isfinite(c->softcap)) return GPT_E_INVALID_ARG;
  if (!(c->rope_base > 0.f) || !isfinite(c->rope_base)) return GPT_E_INVALID_ARG;
  if (!(c->attn_scale > 0.f) || !isfinite(c->attn_scale)) return GPT_E_INVALID_ARG;
  if (!(c->norm_eps >= 0.f) || !isfinite(c->norm_eps)) return GPT_E_INVALID_ARG;
  // Limits of what the kernels implement.
  const long M = (long)c->batch * c->seq_len;
  if (M > (1L << 30) || (long)c->vocab * c->d_model > (1L << 31)) return GPT_E_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return GPT_E_UNSUPPORTED;
  if (c->d_model % 64 || c->mlp_dim % 64 || (c->n_head * c->head_dim) % 64) return GPT_E_UNSUPPORTED;
  if (c->d_model > 8192) return GPT_E_UNSUPPORTED;
  if (!rope_fits(c->seq_len, c->head_dim)) return GPT_E_UNSUPPORTED;
  if (c->dtype == GPT_BF16) {
    if (c->seq_len % 64) return GPT_E_UNSUPPORTED;
    if (!attn_bf16_fits(c->seq_len, c->n_head, c->n_kv_head, c->head_dim)) return GPT_E_UNSUPPORTED;
    if ((c->n_head * c->head_dim) % 128 || (c->n_kv_head * c->head_dim) % 128) return GPT_E_UNSUPPORTED;
  }
  if (any_ve(c)) {
    if (c->d_model < VE_GATE_CH) return GPT_E_UNSUPPORTED;
    if (c->dtype == GPT_BF16 && c->head_dim != 128) return GPT_E_UNSUPPORTED;  // fused epilogue only
  }
  if (c->looped != 0 && c->looped != 1) return GPT_E_INVALID_ARG;
  if (c->looped && c->dtype == GPT_BF16 && c->head_dim != 128) return GPT_E_UNSUPPORTED;
  if (c->nested_c1 != 0) {
    const long c1 = c->nested_c1, C = c->d_model;
    if (c1 < 0 || c1 > C) return GPT_E_INVALID_ARG;
    // every partitioned dimension splits exactly in the proportion c1 : C
    if ((c->n_head * c1) % C || (c->n_kv_head * c1) % C || (c->mlp_dim * c1) % C)
      return GPT_E_INVALID_ARG;
    if (c->looped || any_ve(c)) return GPT_E_UNSUPPORTED;
    if (c1 % 64 || (c->mlp_dim * c1 / C) % 64) return GPT_E_UNSUPPORTED;
    if (c->dtype == GPT_BF16 && ((c->n_head * c1 / C * c->head_dim) % 128 ||
                                 (c->n_kv_head * c1 / C * c->head_dim) % 128))
      return GPT_E_UNSUPPORTED;
  }
  return GPT_OK;
}

// Shares of the inner block of a nested model (validated exact).
struct Split {
  int c1, h1, hkv1, f1;
};
Split split_of(const gpt_cfg* c) {
  const long c1 = c->nested_c1, C = c->d_model;
  return {(int)c1, (int)(c->n_head * c1 / C), (int)(c->n_kv_head * c1 / C), (int)(c->mlp_dim * c1 / C)};
}

Layout plan(const gpt_cfg* c) {
  Layout L{};
  const size_t M = (size_t)c->batch * c->seq_len;
  const size_t C = c->d_model, H = c->n_head, Hkv = c->n_kv_head, D = c->head_dim, F = c->mlp_dim;
  const bool bf = c->dtype == GPT_BF16;
  const size_t es = bf ? 2 : 4;
  L.nnb = bf ? gemm_bf16_ce_blocks(c->vocab) : gemm_f32_ce_blocks(c->vocab);
  size_t off = 0;
  L.flags = off; off += up(64);
  L.x = off; off += up(M * C * 4);
  L.x0 = off; off += up(M * C * 4);
  L.xn = off; off += up(M * C * es);
  if (bf) {
    L.qk = off; off += up(M * (H + Hkv) * D * 2);
    L.vt = off; off += up(M * Hkv * D * 2);
  } else {
    L.qk = off; off += up(M * (H + 2 * Hkv) * D * 4);
    L.vt = off;
  }
  L.o = off; off += up(M * H * D * es);
  L.h = off; off += up(M * F * es);
  L.cs = off; off += up((size_t)c->seq_len * (D / 2) * 8);
  L.ssp = off; off += up(M * (size_t)(C / 64) * 4);  // slices are >= 64 columns wide
  L.partial = off; off += up(M * (size_t)L.nnb * 4);
  L.tgt = off; off += up(M * 4);
  // looped trunk: every pass-1 layer's q, k (bf16: the qk layout; fp32: the whole qkv rows)
  L.qk1 = off;
  if (c->looped) off += up((size_t)c->n_layer * M * (bf ? (H + Hkv) * D * 2 : (H + 2 * Hkv) * D * 4));
  L.last = off; off += up((size_t)c->batch * C * 4);  // prefill: each row's last position, normed
  // nested bf16: the kfront=1 cross-entropy sums taken inside the lm_head pass (per row, column
  // block and wavefront) and the kfront=1 target logits
  L.partial1 = off;
  L.tgt1 = off;
  if (c->nested_c1 && bf) {
    off += up(M * (size_t)L.nnb * 4 * 4);
    L.tgt1 = off; off += up(M * 4);
  }
  L.total = off;
  return L;
}

#define CK(expr)                                 \
  do {                                           \
    if ((expr) != hipSuccess) return GPT_E_HIP;  \
  } while (0)

GemmArgs gemm_args(const void* A, int lda, const void* B, int N, int K, int M, void* out, int ldo) {
  GemmArgs g{};
  g.A = A; g.lda = lda;
  g.B0 = B; g.B1 = B; g.B2 = B; g.nseg0 = N; g.nseg1 = 0; g.ldb = K;
  g.M = M; g.N = N; g.K = K;
  g.out = out; g.ldo = ldo;
  return g;
}

hipError_t gemm(bool bf, Epi e, const GemmArgs& g, hipStream_t s) {
  return bf ? launch_gemm_bf16(e, g, s) : launch_gemm_f32(e, g, s);
}

// Launch timing (gpt_fwd_loss_timed): pair `recorded` of the caller's events takes the start
// of the first and the end of the last kernel enqueued at one launch site of the requested kind
// (hipExtLaunchKernelGGL stamps them from the dispatch itself), while pairs remain.
struct Timer {
  gpt_launch_timing* t;
  bool on(int kind) const { return t && t->kind == kind && t->recorded < t->capacity; }
  void begin(int kind) const {
    if (on(kind)) launch_events = {(hipEvent_t)t->begin[t->recorded], (hipEvent_t)t->end[t->recorded]};
  }
  void end(int kind) const {
    if (on(kind)) { launch_events = {}; ++t->recorded; }
  }
};
// Enqueue `call` (a hipError_t expression) inside the timer's window; the window is closed
// before an error returns.
#define TIMED(tm, kind, call)                        \
  do {                                               \
    (tm).begin(kind);                                \
    const hipError_t timed_err_ = (call);            \
    (tm).end(kind);                                  \
    if (timed_err_ != hipSuccess) return GPT_E_HIP;  \
  } while (0)

// lm_head + softcap + CE over M rows into loss/mean (targets may be NULL: logits only).  If
// rs_ssp is set, xf is the un-normalised stream and the GEMM applies the final RMSNorm as a row
// scale from those per-slice sums of squares.
gpt_status lm_head_ce(bool bf, const void* xf, const void* wu, const int32_t* targets,
                      const int32_t* tokens, int M, int C, int V, float cap, float* loss,
                      float* mean, float* logits, float* partial, float* tgt, int nnb,
                      unsigned* flags, hipStream_t s, const Timer& tm, const float* rs_ssp = nullptr,
                      float eps = 0.f, int K = 0) {
  // K < C: the product over input columns [0, K) only (xf and wu keep their row stride C)
  if (K <= 0) K = C;
  GemmArgs g = gemm_args(xf, C, wu, V, K, M, nullptr, 0);
  g.ldb = C;
  if (rs_ssp) { g.rs_ssp = rs_ssp; g.rs_n = C / gemm_resid_slice_cols(M, C); g.rs_c = (float)C; g.eps = eps; }
  g.targets = targets; g.partial = partial; g.tgt_logit = tgt; g.logits = logits;
  g.nnb = nnb; g.cap = cap;
  TIMED(tm, GPT_KERNEL_LM_HEAD, gemm(bf, EPI_CE, g, s));
  if (logits && !bf) CK(launch_softcap(logits, (size_t)M * V, cap, s));  // bf16: written softcapped
  if (targets) {
    CK(launch_ce_finalize(partial, nnb, tgt, targets, tokens, M, V, cap, loss, flags, s));
    CK(launch_ce_mean(loss, targets, M, mean, s));
  }
  return GPT_OK;
}

// Row block r (0 or 1) of a nested linear [out, in] with inner shares (o1, i1): its first
// element (row block 2 follows row block 1).
const void* row_block(const void* base, int r, int o1, int i1, size_t es) {
  return r == 0 ? base : (const char*)base + (size_t)o1 * i1 * es;
}

// The layers of a nested (two-block) model, from the embedding to the final PrefixRMSNorm'd
// stream in xn ("Fully Nested Transformers", opening section: block lower triangular linears
// and PrefixRMSNorm).  Row block 1 of every linear is a GEMM over the inner input columns
// [0, in1) writing the inner output columns; row block 2 a GEMM over all input columns writing
// the rest.  Each output element is written by exactly one of the two, so residual epilogues
// (and the next layer's x0 mix in the MLP down-projection) apply per element unchanged.  Every
// norm is materialised by the row kernel (a PrefixRMSNorm is not a row scale of the product).
gpt_status nested_layers(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
                         const Split& sp, const Layout& L, char* ws, const Timer& tm,
                         hipStream_t s) {
  const bool bf = c->dtype == GPT_BF16;
  const size_t es = bf ? 2 : 4;
  const int B = c->batch, T = c->seq_len, M = B * T, C = c->d_model, H = c->n_head;
  const int Hkv = c->n_kv_head, D = c->head_dim, F = c->mlp_dim, V = c->vocab;
  const int c1 = sp.c1, h1 = sp.h1, hkv1 = sp.hkv1, f1 = sp.f1;
  const float eps = c->norm_eps;
  unsigned* flags = (unsigned*)(ws + L.flags);
  float* x = (float*)(ws + L.x);
  float* x0 = (float*)(ws + L.x0);
  void* xn = ws + L.xn;
  void* qk = ws + L.qk;
  void* vt = ws + L.vt;
  void* o = ws + L.o;
  void* hbuf = ws + L.h;
  const float2* cs = (const float2*)(ws + L.cs);
  float* ssp = (float*)(ws + L.ssp);
  const int nqk = (H + Hkv) * D, nqkv = (H + 2 * Hkv) * D;
  // row block 1 (inner, g1) and row block 2 (outer, g2) of a linear: bf16 runs them as one
  // grouped launch with the outer (longer-K) tiles dispatched first
  auto gemm2 = [&](Epi e, const GemmArgs& g1, const GemmArgs& g2) -> hipError_t {
    if (bf) return launch_gemm_bf16_pair(e, g2, g1, s);
    hipError_t r = g1.N > 0 ? gemm(bf, e, g1, s) : hipSuccess;
    if (r == hipSuccess && g2.N > 0) r = gemm(bf, e, g2, s);
    return r;
  };
  // bf16: every PrefixRMSNorm after the embedding's is applied inside the GEMMs that consume it.
  // The residual pairs (out-projection, MLP down) write bf16(x) and per-slice sums of squares
  // (slices of sw columns; c1 is a whole number of slices); the inner row block of a consumer
  // takes the prefix's RMS as a row scale, the outer one the two-part scale (GemmArgs::pre_k).
  // The final norm, which the lm_head reads for both logits, is materialised.
  int sw = 0;
  if (bf) {
    const GemmArgs a = gemm_args(o, H * D, w->wo[0], c1, h1 * D, M, x, C);
    const GemmArgs b = gemm_args(o, H * D, w->wo[0], C - c1, H * D, M, x + c1, C);
    sw = gemm_pair_resid_slice_cols(a, b);
    if (sw <= 0 || c1 % sw || (C - c1) % sw) sw = 0;  // materialised norms instead
  }
  const bool fused = sw > 0;
  // row scales of the two row blocks of a consumer of the (un-normalised) stream
  auto scale_pair = [&](GemmArgs& in1, GemmArgs& in2) {
    in1.rs_ssp = ssp; in1.rs_n = c1 / sw; in1.rs_c = (float)c1; in1.eps = eps;
    in2.rs_ssp = ssp; in2.rs_n = C / sw; in2.rs_c = (float)C; in2.eps = eps;
    in2.pre_k = c1; in2.pre_n = c1 / sw; in2.pre_c = (float)c1;
  };
  CK(launch_embed_norm(tokens, w->wte, bf, w->resid_lambda, w->x0_lambda, x0, x, xn, M, C, V,
                       eps, flags, s, nullptr, c1));
  for (int l = 0; l < c->n_layer; ++l) {
    const int win = c->window[l] < T ? c->window[l] : T;
    const void* wq[2] = {row_block(w->wq[l], 0, h1 * D, c1, es), row_block(w->wq[l], 1, h1 * D, c1, es)};
    const void* wk[2] = {row_block(w->wk[l], 0, hkv1 * D, c1, es), row_block(w->wk[l], 1, hkv1 * D, c1, es)};
    const void* wv[2] = {row_block(w->wv[l], 0, hkv1 * D, c1, es), row_block(w->wv[l], 1, hkv1 * D, c1, es)};
    const void* wo[2] = {row_block(w->wo[l], 0, c1, h1 * D, es), row_block(w->wo[l], 1, c1, h1 * D, es)};
    const void* w1[2] = {row_block(w->w1[l], 0, f1, c1, es), row_block(w->w1[l], 1, f1, c1, es)};
    const void* w2[2] = {row_block(w->w2[l], 0, c1, f1, es), row_block(w->w2[l], 1, c1, f1, es)};
    if (bf) {
      // q/k/v: one GEMM per row block over its three segments; the epilogue places q and k
      // heads at their model-wide columns and v heads at their model-wide head index
      GemmArgs g[2];
      for (int r = 0; r < 2; ++r) {
        const int hq = r ? H - h1 : h1, hk = r ? Hkv - hkv1 : hkv1;
        g[r] = gemm_args(xn, C, wq[r], (hq + 2 * hk) * D, r ? C : c1, M, qk, nqk);
        g[r].B1 = wk[r]; g[r].B2 = wv[r]; g[r].nseg0 = hq * D; g[r].nseg1 = hk * D;
        g[r].vt = vt; g[r].T = T; g[r].D = D; g[r].Hkv = Hkv; g[r].nqk = (hq + hk) * D; g[r].eps = eps;
        g[r].q_off = r ? h1 * D : 0;
        g[r].k_off = H * D + (r ? hkv1 * D : 0);
        g[r].v_head_off = r ? hkv1 : 0;
        g[r].cs = cs;  // fused RoPE + QK-norm (head_dim 64 or 128)
      }
      if (fused && l > 0) scale_pair(g[0], g[1]);  // layer 0 reads the embedding's normed stream
      TIMED(tm, GPT_KERNEL_QKV, gemm2(EPI_QKV, g[0], g[1]));
      TIMED(tm, GPT_KERNEL_ATTENTION, launch_attn_bf16(qk, vt, o, B, T, H, Hkv, D, win,
                                                       c->attn_scale, s));
    } else {
      // q/k/v into the [q | k | v] rows: one GEMM per (projection, row block)
      const void* wp[3][2] = {{wq[0], wq[1]}, {wk[0], wk[1]}, {wv[0], wv[1]}};
      const int n1[3] = {h1 * D, hkv1 * D, hkv1 * D}, n[3] = {H * D, Hkv * D, Hkv * D};
      const int base[3] = {0, H * D, (H + Hkv) * D};
      for (int j = 0; j < 3; ++j) {
        float* out = (float*)qk + base[j];
        CK(gemm2(EPI_STORE, gemm_args(xn, C, wp[j][0], n1[j], c1, M, out, nqkv),
                 gemm_args(xn, C, wp[j][1], n[j] - n1[j], C, M, out + n1[j], nqkv)));
      }
      CK(launch_qk_rope_norm(qk, false, nqkv, cs, M, T, H + Hkv, D, eps, s));
      CK(launch_attn_f32((const float*)qk, (float*)o, B, T, H, Hkv, D, win, c->attn_scale, s));
    }
    // x += o W_O^T: inner rows read the inner heads' outputs
    GemmArgs go[2] = {gemm_args(o, H * D, wo[0], c1, h1 * D, M, x, C),
                      gemm_args(o, H * D, wo[1], C - c1, H * D, M, x + c1, C)};
    if (fused)
      for (int r = 0; r < 2; ++r) {
        const int c0 = r ? c1 : 0;
        go[r].xb = (bf16_t*)xn + c0; go[r].ssp = ssp; go[r].col_off = c0;
      }
    TIMED(tm, GPT_KERNEL_ATTN_OUT, gemm2(EPI_RESID, go[0], go[1]));
    if (!fused) CK(launch_mix_norm(x, x0, w->resid_lambda, w->x0_lambda, l, false, xn, bf, M, C, eps, s, c1));
    // h = relu(xn W_1^T)^2
    char* hb = (char*)hbuf;
    GemmArgs gu[2] = {gemm_args(xn, C, w1[0], f1, c1, M, hb, F),
                      gemm_args(xn, C, w1[1], F - f1, C, M, hb + (size_t)f1 * es, F)};
    if (fused) scale_pair(gu[0], gu[1]);
    TIMED(tm, GPT_KERNEL_MLP_UP, gemm2(EPI_RELU2, gu[0], gu[1]));
    // x += h W_2^T; the bf16 epilogue also applies the next layer's x0 mix
    const bool more = l + 1 < c->n_layer;
    GemmArgs gd[2] = {gemm_args(hbuf, F, w2[0], c1, f1, M, x, C),
                      gemm_args(hbuf, F, w2[1], C - c1, F, M, x + c1, C)};
    if (bf && more)
      for (int r = 0; r < 2; ++r) {
        const int c0 = r ? c1 : 0;  // first output column of the launch
        gd[r].xb = (bf16_t*)xn + c0; gd[r].ssp = ssp; gd[r].col_off = c0;
        gd[r].x0 = x0 + c0; gd[r].lam = w->resid_lambda; gd[r].mu = w->x0_lambda; gd[r].layer = l + 1;
      }
    TIMED(tm, GPT_KERNEL_MLP_DOWN, gemm2(EPI_RESID, gd[0], gd[1]));
    if (!fused || !more)
      CK(launch_mix_norm(x, x0, w->resid_lambda, w->x0_lambda, l + 1, more && !bf, xn, bf, M, C, eps,
                         s, c1));
  }
  return GPT_OK;
}

gpt_status run(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
               const int32_t* targets, float* loss, float* mean_loss, float* logits,
               float* loss1, float* mean1, float* logits1, void* workspace,
               size_t workspace_bytes, void* stream, gpt_launch_timing* timing,
               const Prefill* pf = nullptr);

}  // namespace

extern "C" {

gpt_status gpt_validate(const gpt_cfg* cfg) { return validate(cfg); }

size_t gpt_workspace_bytes(const gpt_cfg* cfg) {
  if (validate(cfg) != GPT_OK) return 0;
  return plan(cfg).total;
}

gpt_status gpt_fwd_loss(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
                        const int32_t* targets, float* loss, float* mean_loss, float* logits,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return gpt_fwd_loss_timed(c, w, tokens, targets, loss, mean_loss, logits, workspace,
                            workspace_bytes, stream, nullptr);
}

gpt_status gpt_fwd_loss_timed(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
                              const int32_t* targets, float* loss, float* mean_loss,
                              float* logits, void* workspace, size_t workspace_bytes,
                              void* stream, gpt_launch_timing* timing) {
  return run(c, w, tokens, targets, loss, mean_loss, logits, nullptr, nullptr, nullptr, workspace,
             workspace_bytes, stream, timing);
}

gpt_status gpt_fwd_loss_nested(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
                               const int32_t* targets, float* loss, float* mean_loss,
                               float* logits, float* loss_k1, float* mean_k1, float* logits_k1,
                               void* workspace, size_t workspace_bytes, void* stream,
                               gpt_launch_timing* timing) {
  if (!c || c->nested_c1 == 0) return GPT_E_INVALID_ARG;
  return run(c, w, tokens, targets, loss, mean_loss, logits, loss_k1, mean_k1, logits_k1,
             workspace, workspace_bytes, stream, timing);
}

}  // extern "C"

namespace {

gpt_status run(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
               const int32_t* targets, float* loss, float* mean_loss, float* logits,
               float* loss1, float* mean1, float* logits1, void* workspace,
               size_t workspace_bytes, void* stream, gpt_launch_timing* timing,
               const Prefill* pf) {
  if (timing) {
    if (timing->kind < GPT_KERNEL_QKV || timing->kind > GPT_KERNEL_LM_HEAD || timing->capacity < 0 ||
        (timing->capacity > 0 && (!timing->begin || !timing->end)))
      return GPT_E_INVALID_ARG;
    timing->recorded = 0;
  }
  gpt_status st = validate(c);
  if (st != GPT_OK) return st;
  if (!w || !tokens) return GPT_E_INVALID_ARG;
  if (!w->wte || !w->lm_head || !w->resid_lambda || !w->x0_lambda || !w->wq || !w->wk || !w->wv ||
      !w->wo || !w->w1 || !w->w2)
    return GPT_E_INVALID_ARG;
  for (int l = 0; l < c->n_layer; ++l)
    if (!w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->w1[l] || !w->w2[l])
      return GPT_E_INVALID_ARG;
  if (any_ve(c)) {
    if (!w->ve || !w->ve_gate) return GPT_E_INVALID_ARG;
    for (int l = 0; l < c->n_layer; ++l)
      if (c->has_ve[l] && (!w->ve[l] || !w->ve_gate[l] || !aligned(w->ve[l], 16) ||
                           !aligned(w->ve_gate[l], 4)))
        return GPT_E_INVALID_ARG;
  }
  if (c->looped && (!w->pass_emb || !w->gate_logit || !aligned(w->pass_emb, 16) ||
                    !aligned(w->gate_logit, 4)))
    return GPT_E_INVALID_ARG;
  if (targets && (!loss || !mean_loss)) return GPT_E_INVALID_ARG;
  if (!targets && !logits && !pf) return GPT_E_INVALID_ARG;
  if (!loss1 != !mean1 || (loss1 && !targets) || (loss1 && !aligned(loss1, 4)) ||
      (mean1 && !aligned(mean1, 4)) || (logits1 && !aligned(logits1, 4)))
    return GPT_E_INVALID_ARG;
  const bool want1 = loss1 || logits1;
  const void* ptrs16[] = {w->wte, w->lm_head};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return GPT_E_INVALID_ARG;
  for (int l = 0; l < c->n_layer; ++l)
    if (!aligned(w->wq[l], 16) || !aligned(w->wk[l], 16) || !aligned(w->wv[l], 16) ||
        !aligned(w->wo[l], 16) || !aligned(w->w1[l], 16) || !aligned(w->w2[l], 16))
      return GPT_E_INVALID_ARG;
  if (!aligned(tokens, 4) || (targets && !aligned(targets, 4)) || (loss && !aligned(loss, 4)) ||
      (logits && !aligned(logits, 4)))
    return GPT_E_INVALID_ARG;
  const Layout L = plan(c);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, ALIGN)) return GPT_E_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  const Timer tm{timing};
  const bool bf = c->dtype == GPT_BF16;
  const int B = c->batch, T = c->seq_len, M = B * T, C = c->d_model, H = c->n_head;
  const int Hkv = c->n_kv_head, D = c->head_dim, F = c->mlp_dim, V = c->vocab;
  const float eps = c->norm_eps;
  char* ws = (char*)workspace;
  unsigned* flags = (unsigned*)(ws + L.flags);
  float* x = (float*)(ws + L.x);
  float* x0 = (float*)(ws + L.x0);
  void* xn = ws + L.xn;
  void* qk = ws + L.qk;
  void* vt = ws + L.vt;
  void* o = ws + L.o;
  void* hbuf = ws + L.h;
  float2* cs = (float2*)(ws + L.cs);
  float* partial = (float*)(ws + L.partial);
  float* tgt = (float*)(ws + L.tgt);

  CK(launch_clear_u32(flags, 16, s));
  CK(launch_rope_table(cs, T, D, c->rope_base, s));
  const int nqk = (H + Hkv) * D;
  const int nqkv = (H + 2 * Hkv) * D;
  float* ssp = (float*)(ws + L.ssp);
  const int nsl = C / gemm_resid_slice_cols(M, C);  // slices the residual GEMMs write
  // The looped trunk runs two passes: pass 0 keeps every layer's q, k in the qk1 cache (and
  // stops after the last layer's projection, the only part of it pass 2 reads); pass 1 adds
  // the layer's cached prior to its attention logits.  Otherwise there is one pass.
  const size_t es = bf ? 2 : 4;
  if (c->nested_c1) {
    const Split sp = split_of(c);
    if (gpt_status e = nested_layers(c, w, tokens, sp, L, ws, tm, s); e != GPT_OK) return e;
    // The final (prefix-)normalised stream is in xn.  Its first c1 columns are RMSNorm of the
    // inner model's stream, so the product over K in [0, c1) is the kfront=1 logits and the one
    // over all K the full model's: one lm_head pass (bf16, losses only) takes the kfront=1
    // cross-entropy sums when its main loop reaches K = c1.  With logits requested, two passes.
    if (bf && loss1 && !logits && !logits1 && sp.c1 < C) {
      float* partial1 = (float*)(ws + L.partial1);
      float* tgt1 = (float*)(ws + L.tgt1);
      GemmArgs g = gemm_args(xn, C, w->lm_head, V, C, M, nullptr, 0);
      g.ldb = C;
      g.targets = targets; g.partial = partial; g.tgt_logit = tgt; g.nnb = L.nnb; g.cap = c->softcap;
      g.partial1 = partial1; g.nnb1 = 4 * L.nnb; g.pre_k = sp.c1;
      TIMED(tm, GPT_KERNEL_LM_HEAD, launch_gemm_bf16(EPI_CE, g, s));
      CK(launch_prefix_target_logit(xn, w->lm_head, targets, M, C, sp.c1, V, tgt1, s));
      CK(launch_ce_finalize(partial, L.nnb, tgt, targets, tokens, M, V, c->softcap, loss, flags, s));
      CK(launch_ce_mean(loss, targets, M, mean_loss, s));
      CK(launch_ce_finalize(partial1, 4 * L.nnb, tgt1, targets, tokens, M, V, c->softcap, loss1, flags, s));
      CK(launch_ce_mean(loss1, targets, M, mean1, s));
      return GPT_OK;
    }
    gpt_status e = lm_head_ce(bf, xn, w->lm_head, targets, tokens, M, C, V, c->softcap, loss,
                              mean_loss, logits, partial, tgt, L.nnb, flags, s, tm);
    if (e != GPT_OK || !want1) return e;
    return lm_head_ce(bf, xn, w->lm_head, loss1 ? targets : nullptr, tokens, M, C, V, c->softcap,
                      loss1, mean1, logits1, partial, tgt, L.nnb, flags, s, tm, nullptr, 0.f, sp.c1);
  }
  const size_t qk1_layer = (size_t)M * (bf ? nqk : nqkv) * es;
  for (int pass = c->looped ? 0 : 1; pass < 2; ++pass) {
    const bool capture = c->looped && pass == 0, prior = c->looped && pass == 1;
    const void* pe = c->looped ? (const char*)w->pass_emb + (size_t)pass * C * es : nullptr;
    CK(launch_embed_norm(tokens, w->wte, bf, w->resid_lambda, w->x0_lambda, x0, x, xn, M, C, V,
                         eps, flags, s, pe));
    for (int l = 0; l < c->n_layer; ++l) {
      void* qk_l = capture ? (void*)(ws + L.qk1 + l * qk1_layer) : qk;
      const void* qk1_l = prior ? (const void*)(ws + L.qk1 + l * qk1_layer) : nullptr;
      const float* gl = prior ? w->gate_logit : nullptr;
      const int win = c->window[l] < T ? c->window[l] : T;
      if (bf) {
        // bf16: every RMSNorm after the first is applied as a row scale inside the GEMM that
        // consumes it (RMSNorm(x) W^T = (x W^T) / rms(x)).  The residual epilogues keep x in
        // fp32, apply the next layer's x0 mix, and emit bf16(x) plus per-slice sums of squares.
        bf16_t* xb = (bf16_t*)xn;
        GemmArgs g = gemm_args(xn, C, w->wq[l], nqkv, C, M, qk_l, nqk);
        g.B1 = w->wk[l]; g.B2 = w->wv[l]; g.nseg0 = H * D; g.nseg1 = Hkv * D; g.k_off = H * D;
        g.vt = vt; g.T = T; g.D = D; g.Hkv = Hkv; g.nqk = nqk; g.eps = eps;
        g.cs = cs;  // RoPE + QK-norm in the GEMM epilogue (head_dim 64 or 128)
        if (l > 0) { g.rs_ssp = ssp; g.rs_n = nsl; g.rs_c = (float)C; }  // layer 0 reads normed xn
        if (c->has_ve && c->has_ve[l]) {  // validated: D == 128, so the fused epilogue adds it
          g.ve = (const bf16_t*)w->ve[l]; g.ve_gate = (const bf16_t*)w->ve_gate[l];
          g.tokens = tokens; g.vocab = V;
        }
        TIMED(tm, GPT_KERNEL_QKV, launch_gemm_bf16(EPI_QKV, g, s));
        if (pf) {
          char* kc = (char*)pf->cache + (size_t)l * 2 * B * Hkv * pf->T * D * 2;
          CK(launch_cache_fill(true, qk_l, nqk, H * D, vt, 0, B, T, pf->T, Hkv, D, kc,
                               kc + (size_t)B * Hkv * pf->T * D * 2, s));
        }
        if (capture && l + 1 == c->n_layer) break;
        TIMED(tm, GPT_KERNEL_ATTENTION, launch_attn_bf16(qk_l, vt, o, B, T, H, Hkv, D, win,
                                                         c->attn_scale, s, qk1_l, gl, l));
        // x += o W_O^T, then bf16(x) and sums of squares for the MLP's norm
        GemmArgs go = gemm_args(o, H * D, w->wo[l], C, H * D, M, x, C);
        go.xb = xb; go.ssp = ssp; go.ssp_n = nsl;
        TIMED(tm, GPT_KERNEL_ATTN_OUT, launch_gemm_bf16(EPI_RESID, go, s));
        // h = relu(RMSNorm(x) W_1^T)^2
        GemmArgs gu = gemm_args(xb, C, w->w1[l], F, C, M, hbuf, F);
        gu.rs_ssp = ssp; gu.rs_n = nsl; gu.rs_c = (float)C; gu.eps = eps;
        TIMED(tm, GPT_KERNEL_MLP_UP, launch_gemm_bf16(EPI_RELU2, gu, s));
        // x += h W_2^T, then the next layer's x0 mix (if any), bf16(x) and sums of squares
        GemmArgs gd = gemm_args(hbuf, F, w->w2[l], C, F, M, x, C);
        gd.xb = xb; gd.ssp = ssp; gd.ssp_n = nsl;
        if (l + 1 < c->n_layer) { gd.x0 = x0; gd.lam = w->resid_lambda; gd.mu = w->x0_lambda; gd.layer = l + 1; }
        TIMED(tm, GPT_KERNEL_MLP_DOWN, launch_gemm_bf16(EPI_RESID, gd, s));
      } else {
        // q, k, v projections (one GEMM over the three weight segments)
        GemmArgs g = gemm_args(xn, C, w->wq[l], nqkv, C, M, qk_l, nqkv);
        g.B1 = w->wk[l]; g.B2 = w->wv[l]; g.nseg0 = H * D; g.nseg1 = Hkv * D;
        CK(launch_gemm_f32(EPI_STORE, g, s));
        if (c->has_ve && c->has_ve[l])
          CK(launch_ve_mix_f32((float*)qk_l, nqkv, nqk, (const float*)xn, C, tokens, V,
                               (const float*)w->ve[l], (const float*)w->ve_gate[l], M, Hkv, D, s));
        // RoPE + QK-norm on the q and k heads
        CK(launch_qk_rope_norm(qk_l, false, nqkv, cs, M, T, H + Hkv, D, eps, s));
        if (pf) {
          char* kc = (char*)pf->cache + (size_t)l * 2 * B * Hkv * pf->T * D * 4;
          CK(launch_cache_fill(false, qk_l, nqkv, H * D, qk_l, (H + Hkv) * D, B, T, pf->T, Hkv, D,
                               kc, kc + (size_t)B * Hkv * pf->T * D * 4, s));
        }
        if (capture && l + 1 == c->n_layer) break;
        // windowed causal attention
        CK(launch_attn_f32((const float*)qk_l, (float*)o, B, T, H, Hkv, D, win, c->attn_scale, s,
                           (const float*)qk1_l, gl, l));
        // x += o W_O^T
        CK(launch_gemm_f32(EPI_RESID, gemm_args(o, H * D, w->wo[l], C, H * D, M, x, C), s));
        // MLP: x += relu(RMSNorm(x) W_1^T)^2 W_2^T
        CK(launch_mix_norm(x, x0, w->resid_lambda, w->x0_lambda, l, false, xn, false, M, C, eps, s));
        CK(launch_gemm_f32(EPI_RELU2, gemm_args(xn, C, w->w1[l], F, C, M, hbuf, F), s));
        CK(launch_gemm_f32(EPI_RESID, gemm_args(hbuf, F, w->w2[l], C, F, M, x, C), s));
        // next layer's x0 mix and pre-attention norm, or the final norm
        const bool more = l + 1 < c->n_layer;
        CK(launch_mix_norm(x, x0, w->resid_lambda, w->x0_lambda, l + 1, more, xn, false, M, C, eps, s));
      }
    }
  }
  if (pf) {  // logits at each row's last prompt position: its normed row times W_U^T
    void* last = ws + L.last;
    CK(launch_last_row_norm(bf, x, pf->lens, B, T, C, eps, last, flags, s));
    CK(launch_gemv(bf, DEC_LOGITS, last, C, B, w->lm_head, w->lm_head, w->lm_head, V, 0, V, C,
                   pf->logits, V, s, 1, nullptr, c->softcap));
    return GPT_OK;
  }
  if (bf)
    return lm_head_ce(bf, xn, w->lm_head, targets, tokens, M, C, V, c->softcap, loss, mean_loss,
                      logits, partial, tgt, L.nnb, flags, s, tm, ssp, eps);
  return lm_head_ce(bf, xn, w->lm_head, targets, tokens, M, C, V, c->softcap, loss, mean_loss,
                    logits, partial, tgt, L.nnb, flags, s, tm);
}

}  // namespace

extern "C" {

// ------------------------------------------------------------------------------- decoding

static gpt_status validate_decode(const gpt_cfg* c) {
  const gpt_status st = validate(c);
  if (st != GPT_OK) return st;
  if (c->batch > 32 || c->seq_len > 8192 || c->n_head / c->n_kv_head > 8) return GPT_E_UNSUPPORTED;
  // bf16: a product's row scale takes up to 128 per-block row sums (the out-projection leaves
  // d_model / 32 of them); 4096 is also the widest model the decode tests cover
  if (c->dtype == GPT_BF16 && c->d_model > 4096) return GPT_E_UNSUPPORTED;
  if (any_ve(c) || c->looped || c->nested_c1) return GPT_E_UNSUPPORTED;
  return GPT_OK;
}

// K splits of the decode step's products (bf16): the q/k/v projection, the attention output
// projection and the MLP down-projection split K when N alone gives too few blocks; their
// consumers (the RoPE/append kernel, the residual norms) sum the partial tiles.
struct DecodeSplits {
  int qkv, out, down;
};

// bf16: the out-projection does not split K -- it adds into x itself and leaves bf16(x) and
// per-block sums of squares, from which the MLP-up product applies the norm as a row scale.
static DecodeSplits decode_splits(const gpt_cfg* c) {
  if (c->dtype != GPT_BF16) return {1, 1, 1};
  const int C = c->d_model, H = c->n_head, Hkv = c->n_kv_head, D = c->head_dim, F = c->mlp_dim;
  return {gemv_splits((H + 2 * Hkv) * D, C), 1, gemv_splits(C, F)};
}

struct DecodeLayout {
  size_t flags, x, x0, xn, y, q, o, h, part, gpart, ss_o, ss_m, total;
};

static DecodeLayout decode_plan(const gpt_cfg* c) {
  DecodeLayout L{};
  const size_t B = c->batch, C = c->d_model, H = c->n_head, Hkv = c->n_kv_head, D = c->head_dim;
  const size_t F = c->mlp_dim, es = c->dtype == GPT_BF16 ? 2 : 4;
  const DecodeSplits ks = decode_splits(c);
  const size_t ro = (size_t)(ks.out > ks.down ? ks.out : ks.down) * B * C;  // residual partials
  size_t off = 0;
  L.flags = off; off += up(64);
  L.x = off; off += up(B * C * 4);
  L.x0 = off; off += up(B * C * 4);
  L.xn = off; off += up(B * C * es);
  L.y = off; off += up((size_t)ks.qkv * B * (H + 2 * Hkv) * D * 4);
  L.q = off; off += up(B * H * D * es);
  L.o = off; off += up(B * H * D * es);
  L.h = off; off += up(B * F * es);
  L.part = off; off += up(B * H * (size_t)decode_attn_chunks(c->seq_len) * (D + 2) * 4);
  L.gpart = off; off += up(ro * 4);
  L.ss_o = off; off += up(B * ((C + 31) / 32) * 4);               // bf16: out-projection row sums
  L.ss_m = off; off += up(B * (size_t)add_mix_rows_blocks(C) * 4);  // bf16: MLP-down row sums
  L.total = off;
  return L;
}

size_t gpt_kv_cache_bytes(const gpt_cfg* c) {
  if (validate_decode(c) != GPT_OK) return 0;
  const size_t es = c->dtype == GPT_BF16 ? 2 : 4;
  return (size_t)c->n_layer * 2 * c->batch * c->n_kv_head * c->seq_len * c->head_dim * es;
}

size_t gpt_decode_workspace_bytes(const gpt_cfg* c) {
  if (validate_decode(c) != GPT_OK) return 0;
  return decode_plan(c).total;
}

gpt_status gpt_decode_step(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
                           const int32_t* pos, void* kv_cache, float* logits, void* workspace,
                           size_t workspace_bytes, void* stream) {
  gpt_status st = validate_decode(c);
  if (st != GPT_OK) return st;
  if (!w || !tokens || !pos || !logits) return GPT_E_INVALID_ARG;
  if (!w->wte || !w->lm_head || !w->resid_lambda || !w->x0_lambda || !w->wq || !w->wk || !w->wv ||
      !w->wo || !w->w1 || !w->w2)
    return GPT_E_INVALID_ARG;
  for (int l = 0; l < c->n_layer; ++l)
    if (!w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->w1[l] || !w->w2[l] ||
        !aligned(w->wq[l], 16) || !aligned(w->wk[l], 16) || !aligned(w->wv[l], 16) ||
        !aligned(w->wo[l], 16) || !aligned(w->w1[l], 16) || !aligned(w->w2[l], 16))
      return GPT_E_INVALID_ARG;
  if (!aligned(w->wte, 16) || !aligned(w->lm_head, 16) || !aligned(tokens, 4) || !aligned(pos, 4) ||
      !aligned(logits, 4))
    return GPT_E_INVALID_ARG;
  if (!kv_cache || !aligned(kv_cache, ALIGN)) return GPT_E_INVALID_ARG;
  const DecodeLayout L = decode_plan(c);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, ALIGN)) return GPT_E_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  const bool bf = c->dtype == GPT_BF16;
  const int B = c->batch, T = c->seq_len, C = c->d_model, H = c->n_head, Hkv = c->n_kv_head;
  const int D = c->head_dim, F = c->mlp_dim, V = c->vocab;
  const size_t es = bf ? 2 : 4;
  const float eps = c->norm_eps;
  char* ws = (char*)workspace;
  unsigned* flags = (unsigned*)(ws + L.flags);
  float* x = (float*)(ws + L.x);
  float* x0 = (float*)(ws + L.x0);
  void* xn = ws + L.xn;
  float* y = (float*)(ws + L.y);
  void* q = ws + L.q;
  void* o = ws + L.o;
  void* hb = ws + L.h;
  const int nqkv = (H + 2 * Hkv) * D;
  const size_t cache_half = (size_t)B * Hkv * T * D * es;  // k or v of one layer

  float* gpart = (float*)(ws + L.gpart);
  const DecodeSplits ks = decode_splits(c);
  CK(launch_clear_u32(flags, 16, s));
  CK(launch_embed_norm(tokens, w->wte, bf, w->resid_lambda, w->x0_lambda, x0, x, xn, B, C, V, eps,
                       flags, s));
  // bf16: xn holds bf16(x) of the un-normalised stream after layer 0's q/k/v (embed_norm's xn is
  // normalised), and the products that read it apply 1/rms from per-block row sums (ss_o, ss_m).
  float* ss_o = (float*)(ws + L.ss_o);
  float* ss_m = (float*)(ws + L.ss_m);
  const int no = (C + 31) / 32, nm = add_mix_rows_blocks(C);
  for (int l = 0; l < c->n_layer; ++l) {
    char* kc = (char*)kv_cache + (size_t)l * 2 * cache_half;
    char* vc = kc + cache_half;
    const int win = c->window[l] < T ? c->window[l] : T;
    // q/k/v (K-split partials in y), then RoPE + QK-norm and the cache append
    CK(launch_gemv(bf, DEC_STORE, xn, C, B, w->wq[l], w->wk[l], w->wv[l], H * D, Hkv * D, nqkv, C,
                   y, nqkv, s, ks.qkv, y, 0.f, nullptr, nullptr, 0, 0, bf && l > 0 ? ss_m : nullptr, nm,
                   eps));
    CK(launch_rope_append(bf, y, nqkv, ks.qkv, pos, B, T, H, Hkv, D, eps, c->rope_base, q, kc, vc,
                          flags, s));
    CK(launch_decode_attn(bf, q, kc, vc, pos, B, T, H, Hkv, D, win, c->attn_scale, o,
                          (float*)(ws + L.part), s));
    // x += o W_O^T, then h = relu(RMSNorm(x) W_1^T)^2 (bf16: the norm as the MLP-up product's row
    // scale; fp32: xn = RMSNorm(x) by the norm kernel first)
    if (bf) {
      CK(launch_gemv(bf, DEC_RESID_RS, o, H * D, B, w->wo[l], w->wo[l], w->wo[l], C, 0, C, H * D, x, C,
                     s, 1, nullptr, 0.f, nullptr, nullptr, 0, 0, nullptr, 0, 0.f, xn, ss_o));
      CK(launch_gemv(bf, DEC_RELU2, xn, C, B, w->w1[l], w->w1[l], w->w1[l], F, 0, F, C, hb, F, s, 1,
                     nullptr, 0.f, nullptr, nullptr, 0, 0, ss_o, no, eps));
    } else {
      CK(launch_gemv(bf, DEC_RESID, o, H * D, B, w->wo[l], w->wo[l], w->wo[l], C, 0, C, H * D, x, C, s));
      CK(launch_mix_norm(x, x0, w->resid_lambda, w->x0_lambda, l, false, xn, bf, B, C, eps, s));
      CK(launch_gemv(bf, DEC_RELU2, xn, C, B, w->w1[l], w->w1[l], w->w1[l], F, 0, F, C, hb, F, s));
    }
    // x += h W_2^T, then the next layer's x0 mix (bf16: bf16(x) and row sums for the next
    // product; fp32: the norm as well)
    const bool more = l + 1 < c->n_layer;
    if (bf) {
      CK(launch_gemv(bf, DEC_RESID, hb, F, B, w->w2[l], w->w2[l], w->w2[l], C, 0, C, F, x, C, s,
                     ks.down, gpart));
      // (KS = 1: the product has added into x itself and there are no partials)
      CK(launch_add_mix_rows(x, ks.down > 1 ? gpart : nullptr, ks.down > 1 ? ks.down : 0, x0,
                             w->resid_lambda, w->x0_lambda, l + 1, more, xn, ss_m, B, C, s));
    } else {
      CK(launch_gemv(bf, DEC_RESID, hb, F, B, w->w2[l], w->w2[l], w->w2[l], C, 0, C, F, x, C, s));
      CK(launch_mix_norm(x, x0, w->resid_lambda, w->x0_lambda, l + 1, more, xn, bf, B, C, eps, s));
    }
  }
  // logits of the final norm (bf16: as the product's row scale)
  CK(launch_gemv(bf, DEC_LOGITS, xn, C, B, w->lm_head, w->lm_head, w->lm_head, V, 0, V, C, logits,
                 V, s, 1, nullptr, c->softcap, pos, tokens, T, V, bf ? ss_m : nullptr, nm, eps));
  return GPT_OK;
}

size_t gpt_prefill_workspace_bytes(const gpt_cfg* c) {
  if (validate_decode(c) != GPT_OK) return 0;
  return plan(c).total;  // the forward over up to seq_len positions
}

gpt_status gpt_prefill(const gpt_cfg* c, const gpt_weights* w, const int32_t* tokens,
                       int32_t prompt_len, const int32_t* lens, void* kv_cache, float* logits,
                       void* workspace, size_t workspace_bytes, void* stream) {
  gpt_status st = validate_decode(c);
  if (st != GPT_OK) return st;
  if (prompt_len < 1 || prompt_len > c->seq_len) return GPT_E_INVALID_ARG;
  if (!kv_cache || !aligned(kv_cache, ALIGN) || !logits || !aligned(logits, 4) ||
      (lens && !aligned(lens, 4)))
    return GPT_E_INVALID_ARG;
  gpt_cfg f = *c;  // the forward over the prompt positions
  f.seq_len = prompt_len;
  st = validate(&f);
  if (st != GPT_OK) return st;
  if (!workspace || workspace_bytes < gpt_prefill_workspace_bytes(c)) return GPT_E_WORKSPACE;
  const Prefill pf{kv_cache, c->seq_len, lens, logits};
  return run(&f, w, tokens, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
             workspace, workspace_bytes, stream, nullptr, &pf);
}

gpt_status gpt_sample(const float* logits, int32_t batch, int32_t vocab, int32_t top_k,
                      float temperature, const float* u, int32_t* out, void* stream) {
  if (!logits || !u || !out || batch < 1 || vocab < 1) return GPT_E_INVALID_ARG;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return GPT_E_INVALID_ARG;
  if ((long)batch * vocab > (1L << 31)) return GPT_E_UNSUPPORTED;
  CK(launch_sample(logits, batch, vocab, top_k, temperature, u, out, (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_device_status(void* workspace, void* stream) {
  if (!workspace) return GPT_E_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return GPT_E_HIP;
  unsigned f = 0;
  if (hipMemcpy(&f, workspace, sizeof(f), hipMemcpyDeviceToHost) != hipSuccess) return GPT_E_HIP;
  return f ? GPT_E_DEVICE_INPUT : GPT_OK;
}

const char* gpt_status_string(gpt_status s) {
  switch (s) {
    case GPT_OK: return "ok";
    case GPT_E_INVALID_ARG: return "invalid argument";
    case GPT_E_UNSUPPORTED: return "configuration not supported by the kernels";
    case GPT_E_WORKSPACE: return "workspace missing, too small or misaligned";
    case GPT_E_HIP: return "HIP launch or runtime error";
    case GPT_E_DEVICE_INPUT: return "token, target id or position out of range";
  }
  return "unknown status";
}

// ---------------------------------------------------------------------------- component ops

static bool dtype_ok(int32_t d) { return d == GPT_F32 || d == GPT_BF16; }

gpt_status gpt_op_embed_norm(int32_t dtype, const int32_t* tokens, const void* wte, const float* lam,
                             const float* mu, float* x0, float* x, void* xn, int32_t M, int32_t C,
                             int32_t V, float eps, uint32_t* flags, void* stream) {
  if (!dtype_ok(dtype) || !tokens || !wte || !lam || !mu || !x0 || !x || !xn || !flags)
    return GPT_E_INVALID_ARG;
  if (M < 1 || C < 4 || V < 1 || C % 4 || C > 8192 || !(eps >= 0.f)) return GPT_E_INVALID_ARG;
  CK(launch_embed_norm(tokens, wte, dtype == GPT_BF16, lam, mu, x0, x, xn, M, C, V, eps, flags,
                       (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_op_mix_norm(int32_t dtype, float* x, const float* x0, const float* lam,
                           const float* mu, int32_t layer, int32_t mix, void* xn, int32_t M,
                           int32_t C, float eps, void* stream) {
  if (!dtype_ok(dtype) || !x || !xn || (mix && (!x0 || !lam || !mu))) return GPT_E_INVALID_ARG;
  if (M < 1 || C < 4 || C % 4 || C > 8192 || layer < 0 || !(eps >= 0.f)) return GPT_E_INVALID_ARG;
  CK(launch_mix_norm(x, x0, lam, mu, layer, mix != 0, xn, dtype == GPT_BF16, M, C, eps,
                     (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_op_rope_table(float* cs, int32_t T, int32_t D, float base, void* stream) {
  if (!cs || T < 1 || D < 2 || (D & 1) || !(base > 0.f)) return GPT_E_INVALID_ARG;
  if (!rope_fits(T, D)) return GPT_E_UNSUPPORTED;
  CK(launch_rope_table((float2*)cs, T, D, base, (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_op_qk_rope_norm(int32_t dtype, void* qk, int32_t ld, const float* cs, int32_t M,
                               int32_t T, int32_t nheads, int32_t D, float eps, void* stream) {
  if (!dtype_ok(dtype) || !qk || !cs || M < 1 || T < 1 || nheads < 1 || D < 2 || (D & 1) ||
      D > 128 || ld < nheads * D || !(eps >= 0.f))
    return GPT_E_INVALID_ARG;
  CK(launch_qk_rope_norm(qk, dtype == GPT_BF16, ld, (const float2*)cs, M, T, nheads, D, eps,
                         (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_op_linear(int32_t dtype, int32_t epi, const void* a, const void* w, int32_t M,
                         int32_t N, int32_t K, void* out, void* stream) {
  if (!dtype_ok(dtype) || !a || !w || !out || M < 1 || N < 1 || K < 1 || epi < 0 || epi > 2)
    return GPT_E_INVALID_ARG;
  const bool bf = dtype == GPT_BF16;
  if (bf && K % 64) return GPT_E_UNSUPPORTED;
  const Epi e = epi == 0 ? EPI_STORE : epi == 1 ? EPI_RELU2 : EPI_RESID;
  CK(gemm(bf, e, gemm_args(a, K, w, N, K, M, out, N), (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_op_qkv(const void* xn, const void* wq, const void* wk, const void* wv, int32_t B,
                      int32_t T, int32_t C, int32_t H, int32_t Hkv, int32_t D, const float* cs,
                      float eps, void* qk, void* vt, void* stream) {
  if (!xn || !wq || !wk || !wv || !qk || !vt || B < 1 || T < 1 || C < 1 || H < 1 || Hkv < 1 || D < 1 ||
      !(eps >= 0.f))
    return GPT_E_INVALID_ARG;
  if (C % 64 || T % 4 || (H * D) % 128 || (Hkv * D) % 128) return GPT_E_UNSUPPORTED;
  if (cs && T % 32) return GPT_E_UNSUPPORTED;  // fused epilogue: whole heads, 32-row groups
  const int M = B * T, nqk = (H + Hkv) * D, nqkv = (H + 2 * Hkv) * D;
  GemmArgs g = gemm_args(xn, C, wq, nqkv, C, M, qk, nqk);
  g.B1 = wk; g.B2 = wv; g.nseg0 = H * D; g.nseg1 = Hkv * D; g.k_off = H * D;
  g.vt = vt; g.T = T; g.D = D; g.Hkv = Hkv; g.nqk = nqk;
  g.cs = (const float2*)cs; g.eps = eps;
  CK(launch_gemm_bf16(EPI_QKV, g, (hipStream_t)stream));
  return GPT_OK;
}

gpt_status gpt_op_attention(int32_t dtype, const void* qk, const void* vt, void* o, int32_t B,
                            int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t window,
                            float scale, void* stream) {
  if (!dtype_ok(dtype) || !qk || !o || B < 1 || T < 1 || H < 1 || Hkv < 1 || H % Hkv ||
      window < 1 || !(scale > 0.f))
    return GPT_E_INVALID_ARG;
  if (D != 64 && D != 128) return GPT_E_UNSUPPORTED;
  const int win = window < T ? window : T;
  if (dtype == GPT_BF16) {
    if (!vt) return GPT_E_INVALID_ARG;
    if (T % 64 || !attn_bf16_fits(T, H, Hkv, D)) return GPT_E_UNSUPPORTED;
    CK(launch_attn_bf16(qk, vt, o, B, T, H, Hkv, D, win, scale, (hipStream_t)stream));
  } else {
    CK(launch_attn_f32((const float*)qk, (float*)o, B, T, H, Hkv, D, win, scale, (hipStream_t)stream));
  }
  return GPT_OK;
}

size_t gpt_op_lm_head_ce_workspace(int32_t dtype, int32_t M, int32_t V) {
  if (!dtype_ok(dtype) || M < 1 || V < 2) return 0;
  const int nnb = dtype == GPT_BF16 ? gemm_bf16_ce_blocks(V) : gemm_f32_ce_blocks(V);
  return up(64) + up((size_t)M * nnb * 4) + up((size_t)M * 4);
}

gpt_status gpt_op_lm_head_ce(int32_t dtype, const void* xf, const void* wu, const int32_t* targets,
                             const int32_t* tokens, int32_t M, int32_t C, int32_t V, float cap,
                             float* loss, float* mean, float* logits, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype) || !xf || !wu || !tokens || M < 1 || C < 1 || V < 2 || !(cap > 0.f))
    return GPT_E_INVALID_ARG;
  if (targets && (!loss || !mean)) return GPT_E_INVALID_ARG;
  if (!targets && !logits) return GPT_E_INVALID_ARG;
  const bool bf = dtype == GPT_BF16;
  if (bf && C % 64) return GPT_E_UNSUPPORTED;
  const size_t need = gpt_op_lm_head_ce_workspace(dtype, M, V);
  if (!workspace || workspace_bytes < need || !aligned(workspace, ALIGN)) return GPT_E_WORKSPACE;
  const int nnb = bf ? gemm_bf16_ce_blocks(V) : gemm_f32_ce_blocks(V);
  char* ws = (char*)workspace;
  unsigned* flags = (unsigned*)ws;
  float* partial = (float*)(ws + up(64));
  float* tgt = (float*)(ws + up(64) + up((size_t)M * nnb * 4));
  hipStream_t s = (hipStream_t)stream;
  CK(launch_clear_u32(flags, 16, s));
  return lm_head_ce(bf, xf, wu, targets, tokens, M, C, V, cap, loss, mean, logits, partial, tgt, nnb,
                    flags, s, Timer{nullptr});
}

}  // extern "C"
