// Host-side launchers of the gfx950 kernels (C++ linkage, internal to libgptfwd).
// Every launcher enqueues on `stream` and returns hipGetLastError() of the launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gptk {

typedef __bf16 bf16_t;

// Measurement hook: while `stop` is set, every kernel the GEMM and attention launchers enqueue
// goes through hipExtLaunchKernelGGL, which stamps `start` with the start of the first such
// kernel (then `start` is cleared) and `stop` with the end of each, i.e. of the last.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents launch_events;

#define GPTK_LAUNCH(kernel, grid, block, stream, ...)                                        \
  do {                                                                                     \
    if (::gptk::launch_events.stop) {                                                      \
      hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream,                    \
                            ::gptk::launch_events.start, ::gptk::launch_events.stop, 0,      \
                            __VA_ARGS__);                                                  \
      ::gptk::launch_events.start = nullptr;                                               \
    } else {                                                                               \
      hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, __VA_ARGS__);         \
    }                                                                                      \
  } while (0)

// ---- row kernels (k_rows.hip) ------------------------------------------------------------
// cos/sin table cs[t * (D/2) + j] = (cos phi, sin phi), phi = t * base^(-2j/D), in fp64 then fp32.
hipError_t launch_rope_table(float2* cs, int T, int D, float base, hipStream_t s);

// Every norm below takes c1 (0 < c1 <= C, a multiple of 4; 0 means C): with c1 < C it is the
// two-block PrefixRMSNorm -- columns [0, c1) divided by the RMS of columns [0, c1), the rest by
// the RMS of the whole row.  c1 = C (or 0) is the plain RMSNorm.

// x0 = RMSNorm(wte[tokens] (+ pe)); x = lam[0] x0 + mu[0] x0; xn = RMSNorm(x).
// wbf16 selects bf16 (else fp32) embedding storage and xn type; pe (optional, [C], the
// embedding's type) is added to every embedding row before the norm.
hipError_t launch_embed_norm(const int32_t* tokens, const void* wte, bool wbf16, const float* lam,
                             const float* mu, float* x0, float* x, void* xn, int M, int C, int V,
                             float eps, unsigned* flags, hipStream_t s, const void* pe = nullptr,
                             int c1 = 0);

// If mix: x = lam[layer] x + mu[layer] x0 (in place).  Then xn = RMSNorm(x).
hipError_t launch_mix_norm(float* x, const float* x0, const float* lam, const float* mu, int layer,
                           bool mix, void* xn, bool xbf16, int M, int C, float eps, hipStream_t s,
                           int c1 = 0);
// x += sum_k add[k] (add: [ks][M][C] partials, summed in order; ks = 0: none), then if mix: x = lam[layer] x +
// mu[layer] x0 (in place); xb = bf16(x) and ss [M][add_mix_rows_blocks(C)] = per-block sums of
// squares of each row of x (its row scale is applied by the consuming product).
int add_mix_rows_blocks(int C);
hipError_t launch_add_mix_rows(float* x, const float* add, int ks, const float* x0, const float* lam,
                               const float* mu, int layer, bool mix, void* xb, float* ss, int M,
                               int C, hipStream_t s);

// fp32 path value embedding, in place on the v columns of qkv [M][ld] (v head h at column
// voff + h*D): v += 3 sigmoid(xn[m][0:12] . gate[h]) * ve[tokens[m]][h*D : (h+1)*D].
hipError_t launch_ve_mix_f32(float* qkv, int ld, int voff, const float* xn, int ldx,
                             const int32_t* tokens, int vocab, const float* ve, const float* gate,
                             int M, int Hkv, int D, hipStream_t s);

// In place on qk [M][nheads*D] (the q heads then the k heads of each token): RoPE at
// position row % T, then per-head RMSNorm.
hipError_t launch_qk_rope_norm(void* qk, bool bf16, int ld, const float2* cs, int M, int T,
                               int nheads, int D, float eps, hipStream_t s);

// ---- decode step (k_decode.hip) ------------------------------------------------------------
// Products of the decode step: y[b][n] = sum_k act[b][k] W[n][k] for b < B <= 32 (act rows
// lda apart; W the row segments W0 | W1 | W2 split at nseg0, nseg0 + nseg1, multiples of 32;
// K a multiple of 64), then per element: DEC_STORE out_f32 = y; DEC_RELU2 out_act =
// relu(y)^2; DEC_RESID out_f32 += y; DEC_LOGITS out_f32 = cap tanh(y / cap), NaN for rows whose
// pos is outside [0, T) or whose token is outside [0, V).
// DEC_RESID_RS (bf16, KS = 1): x += y, also xb = bf16(x) [B][ldo] and ss [B][N / 32] = per-block
// sums of squares of each row of x, for a consumer's row scale.
enum DecEpi { DEC_STORE = 0, DEC_RELU2 = 1, DEC_RESID = 2, DEC_LOGITS = 3, DEC_RESID_RS = 4 };
// KS > 1 (bf16 only) splits K over KS blocks per row block: the product then only stores its
// KS partial tiles in partial[KS][B][N] (no epilogue) and the consumer sums them in order.
// rs (bf16): act is bf16(x) of an un-normalised x and the outputs of row b (partials included)
// are scaled by (sum_{j < rs_n} rs[b * rs_n + j] / K + eps)^-1/2, rs holding per-block sums of
// squares of row b of x (from DEC_RESID_RS or launch_add_mix_rows), rs_n <= 128.
int gemv_splits(int N, int K);
hipError_t launch_gemv(bool bf16, int kind, const void* act, int lda, int B, const void* W0,
                       const void* W1, const void* W2, int nseg0, int nseg1, int N, int K,
                       void* out, int ldo, hipStream_t s, int KS = 1, float* partial = nullptr,
                       float cap = 0.f, const int32_t* pos = nullptr,
                       const int32_t* tokens = nullptr, int T = 0, int V = 0,
                       const float* rs = nullptr, int rs_n = 0, float eps = 0.f, void* xb = nullptr,
                       float* ss = nullptr);
// RoPE at pos[b] + per-head RMSNorm of the q and k heads of y [KS][B][ldy] (fp32 K-split
// partials summed in order; heads q | k | v), q_hat to qout [B, H*D], k_hat and v to the caches
// [B, Hkv, T, D] at position pos[b]; a row with pos outside [0, T) writes nothing and raises
// GPT_FLAG_BAD_POS.
hipError_t launch_rope_append(bool bf16, const float* y, int ldy, int KS, const int32_t* pos, int B,
                              int T, int H, int Hkv, int D, float eps, float base, void* qout,
                              void* kc, void* vc, unsigned* flags, hipStream_t s);
// o [B, H*D] = attention of q [B, H*D] over cached keys/values [B, Hkv, T, D] at positions
// [max(0, pos - window + 1), pos] of each row; part is scratch of
// B * H * decode_attn_chunks(T) * (D + 2) floats.
int decode_attn_chunks(int T);
hipError_t launch_decode_attn(bool bf16, const void* q, const void* kc, const void* vc,
                              const int32_t* pos, int B, int T, int H, int Hkv, int D, int window,
                              float scale, void* o, float* part, hipStream_t s);
// Prefill: the decode cache [B][Hkv][T][D] from one forward pass over P <= T positions.  k_hat
// rows come from qk [B*P][ld] at column kcol0 + g*D; v from vsrc -- bf16: the forward's
// transposed [B][Hkv][D][P]; fp32: rows of [B*P][ld] at column vcol0 + g*D.
hipError_t launch_cache_fill(bool bf16, const void* qk, int ld, int kcol0, const void* vsrc,
                             int vcol0, int B, int P, int T, int Hkv, int D, void* kc, void* vc,
                             hipStream_t s);
// out [B, C] = RMSNorm of x row b*P + lens[b] - 1 (lens NULL: P); bad lengths -> NaN row + flag.
hipError_t launch_last_row_norm(bool bf16, const float* x, const int32_t* lens, int B, int P, int C,
                                float eps, void* out, unsigned* flags, hipStream_t s);
// One token per row from logits [B, V]: argmax if temperature == 0, else the inverse CDF at
// u[b] of softmax(z / temperature) over the top_k largest logits (ties kept; top_k <= 0 or
// >= V keeps all), in vocabulary order.
hipError_t launch_sample(const float* logits, int B, int V, int top_k, float temperature,
                         const float* u, int32_t* out, hipStream_t s);

// ---- GEMMs (k_gemm.hip) --------------------------------------------------------------------
enum Epi { EPI_STORE = 0, EPI_RELU2 = 1, EPI_RESID = 2, EPI_QKV = 3, EPI_CE = 4 };

struct GemmArgs {
  const void* A; int lda;                 // [M, K] row-major
  const void* B0; const void* B1; const void* B2;  // row segments of B [N, K] (row-major, K contiguous)
  int nseg0, nseg1;                       // rows [0,nseg0) in B0, [nseg0,nseg0+nseg1) in B1, rest in B2
  int ldb;
  int M, N, K;
  void* out; int ldo;                     // STORE/RELU2: act [M, ldo]; RESID: float [M, ldo] (+=); QKV: qk
  void* vt; int T, D, Hkv, nqk;           // QKV (bf16 only): columns >= nqk stored transposed to vt [B][Hkv][D][T]
  // QKV output placement: GEMM column c < nseg0 (q) goes to qk column q_off + c, c in
  // [nseg0, nqk) (k) to k_off + (c - nseg0), v columns to KV head v_head_off + (c - nqk) / D.
  // gemm_args() sets the identity (0, nseg0, 0); nested models launch their blocks separately.
  int q_off, k_off, v_head_off;
  const float2* cs;                       // QKV: if set (head_dim 128), RoPE table [T][D/2] -> the q/k
  float eps;                              //      heads get RoPE + RMSNorm in the epilogue
  // QKV with cs set: if ve is set, every v head h of row m gets
  // + 3 sigmoid(rownorm(A[m][0:12]) . ve_gate[h]) * ve[tokens[m]][h*D : (h+1)*D], where rownorm is
  // the row scale below when rs_ssp is set (else A is already normalised).  Token ids outside
  // [0, vocab) read table row 0 (the embedding pass flags them).
  const bf16_t* ve; const bf16_t* ve_gate; const int32_t* tokens; int vocab;
  // Row scale (consumers of an un-normalised A, bf16 path): if rs_ssp is set, every output row
  // is multiplied by rsqrt(sum_j rs_ssp[j][row] / rs_c + eps) before the epilogue's own work,
  // i.e. the GEMM computes RMSNorm(A) W^T from A and its row sums of squares.
  const float* rs_ssp; int rs_n; float rs_c;
  // Prefix row scale (pair launches only; consumers of a PrefixRMSNorm'd A, nested models): if
  // pre_k > 0 (a multiple of 64, rs_ssp set), the product over input columns [0, pre_k) is scaled
  // by rsqrt(sum_{j < pre_n} rs_ssp[j][row] / pre_c + eps) and the rest by the row scale above.
  int pre_k, pre_n; float pre_c;
  // Residual producer (EPI_RESID, bf16 path): if xb is set, after x += acc the epilogue
  // optionally mixes x = lam[layer] x + mu[layer] x0 (when lam != NULL), stores x, a bf16 copy
  // of x to xb [M, ldo], and per-row sums of squares over each column slice of width
  // w = gemm_resid_slice_cols(N) to ssp[(col_off + col) / w][row] (slice-major, M per slice).
  bf16_t* xb; const float* x0; const float* lam; const float* mu; int layer;
  float* ssp; int ssp_n; int col_off;
  const int32_t* targets;                 // CE: [M] (or NULL)
  float* partial;                         // CE: [M][nnb] sums of exp(zhat - cap) per column block
  float* tgt_logit;                       // CE: [M] raw logit z at the target column
  float* logits;                          // CE: optional [M][N] raw fp32 logits (softcap applied later)
  int nnb;                                // CE: number of column blocks
  float cap;                              // CE: softcap
  // CE (256-row tiles, no logits): if partial1 is set, the cross-entropy terms of the partial
  // product over input columns [0, pre_k) (pre_k a multiple of 64, < K) are also summed, per row
  // and wavefront: partial1[row][nnb1] with nnb1 = 4 * nnb (column block b, wavefront w at
  // 4b + w); the targets' logits of that product are not picked up.
  float* partial1; int nnb1;
};

// bf16 inputs, fp32 accumulation on MFMA.  Returns hipErrorInvalidValue for shapes the
// tiling does not cover (K % 64, segment sizes).
hipError_t launch_gemm_bf16(Epi epi, const GemmArgs& a, hipStream_t s);
// Number of column blocks the CE epilogue of launch_gemm_bf16 produces for N columns.
int gemm_bf16_ce_blocks(int N);
// Width of the column slices whose per-row sums of squares an M x N RESID GEMM with xb set
// writes (ssp [N / width][M]); divides N whenever N % 64 == 0.
int gemm_resid_slice_cols(int M, int N);
// Width of the slices a RESID pair (launch_gemm_bf16_pair with xb set) writes for these two
// GEMMs, or 0 if the pair would run as two separate launches.
int gemm_pair_resid_slice_cols(const GemmArgs& a, const GemmArgs& b);
// fp32 SIMT GEMM (small configurations).
hipError_t launch_gemm_f32(Epi epi, const GemmArgs& a, hipStream_t s);
// bf16: two independent GEMMs (same epilogue kind) in one launch, a's tiles dispatched first
// (give a the longer K); N <= 0 in either runs the other alone.
hipError_t launch_gemm_bf16_pair(Epi epi, const GemmArgs& a, const GemmArgs& b, hipStream_t s);
int gemm_f32_ce_blocks(int N);

// ---- attention (k_attn.hip) ----------------------------------------------------------------
// bf16: q/k from qk [B*T][(H+Hkv)*D] (already RoPE'd and normed), v from vt [B][Hkv][D][T];
// o [B*T][H*D].  D must be 128 or 64, T % 64 == 0.  If qk1 is set (looped pass 2; D == 128),
// every logit also gets softplus(gate_logit[layer]) * <q1, k1> from qk1 (same layout as qk).
hipError_t launch_attn_bf16(const void* qk, const void* vt, void* o, int B, int T, int H, int Hkv,
                            int D, int window, float scale, hipStream_t s, const void* qk1 = nullptr,
                            const float* gate_logit = nullptr, int layer = 0);
// fp32: q/k/v from qkv [B*T][(H+2Hkv)*D]; o [B*T][H*D]; qkv1 as qk1 above (qkv layout).
hipError_t launch_attn_f32(const float* qkv, float* o, int B, int T, int H, int Hkv, int D,
                           int window, float scale, hipStream_t s, const float* qkv1 = nullptr,
                           const float* gate_logit = nullptr, int layer = 0);

// ---- loss (k_loss.hip) ----------------------------------------------------------------------
// loss[row] = cap + log(sum_nb partial[row][nb]) - cap tanh(tgt_logit[row] / cap); 0 where
// target = -1;
// NaN (and a flag bit) for an out-of-range target or token.
hipError_t launch_ce_finalize(const float* partial, int nnb, const float* tgt_logit,
                              const int32_t* targets, const int32_t* tokens, int M, int V, float cap,
                              float* loss, unsigned* flags, hipStream_t s);
// bf16: out[row] = sum_{k < c1} x[row][k] * wu[targets[row]][k] in fp32 (rows C apart; 0 where the
// target is -1 or outside [0, V)): the raw target logit of the product over the first c1 columns.
hipError_t launch_prefix_target_logit(const void* x, const void* wu, const int32_t* targets, int M,
                                      int C, int c1, int V, float* out, hipStream_t s);
// z = cap * tanh(z / cap) in place over n floats.
hipError_t launch_softcap(float* z, size_t n, float cap, hipStream_t s);
// Zero n 32-bit words with a kernel (no memset node, so the call stays graph-capturable).
hipError_t launch_clear_u32(unsigned* p, int n, hipStream_t s);
// mean over rows with target != -1 (NaN if none); fixed-order reduction.
hipError_t launch_ce_mean(const float* loss, const int32_t* targets, int M, float* mean, hipStream_t s);

}  // namespace gptk
