// GEMMs of the forward pass, C = A * B^T with A [M,K] and B [N,K] both K-contiguous (the
// row-major [out, in] weight layout), and fused epilogues:
//   STORE  - round to the activation type                    (QKV of the fp32 path)
//   RELU2  - max(0, c)^2, rounded                             (MLP up-projection)
//   RESID  - x += c into the fp32 residual stream             (attention out-proj, MLP down)
//   QKV    - q/k columns row-major, v columns transposed to [B][Hkv][D][T] (bf16 path)
//   CE     - softcap, per-row partial sum of exp(zhat - cap) per column block, and the target's
//            raw logit; the [M, V] logits are never written unless the caller asks for them
//            (then raw, softcapped afterwards by launch_softcap).
//
// Sources: "The Mathematics of Karpathy's nanochat", sections "Causal Self-Attention"
// (projections, no bias), "Output Projection", "Feed-Forward Network (MLP)" (ReLU^2, 4x),
// "Logit Softcap" and "Cross-Entropy Loss".
//
// bf16 kernel (gfx950): v_mfma_f32_32x32x16_bf16 on 32x32 output tiles, fp32 accumulators.
// Block tile BM x BN x 64, WM x WN wavefronts each owning (BM/WM) x (BN/WN).  Operand tiles
// are staged global -> registers -> LDS, double-buffered, one barrier per 64-wide K step.  LDS
// rows are 64 bf16 = eight 16-byte chunks; chunk c of row r lives at c ^ swz(r) so that the
// 16-byte fragment reads of 8 (or 16) consecutive rows hit distinct banks.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gptk {
namespace {

constexpr int BK = 64;

__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// exp(zhat - cap) for zhat = cap * tanh(z / cap), written without cancellation:
// zhat - cap = -2 cap / (1 + exp(2 z / cap)).
__device__ __forceinline__ float ce_term(float z, float two_over_cap_log2e, float m2cap_log2e) {
  const float e = exp2_fast(z * two_over_cap_log2e);
  return exp2_fast(m2cap_log2e * rcp_fast(1.0f + e));
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int AC = BM * 8 / NT, BC = BN * 8 / NT;  // 16-byte chunks per thread per K step
  static_assert(AC * NT == BM * 8 && BC * NT == BN * 8, "tile/thread mismatch");
  static_assert(FM * 32 == TM && FN * 32 == TN, "wave tile must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) bf16 lds[2 * (BM + BN) * BK];
  bf16* const As = lds;
  bf16* const Bs = lds + 2 * BM * BK;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int M = g.M, N = g.N, K = g.K;

  // Tile order: groups of 8 row-blocks sweep the column blocks, so concurrently resident
  // blocks share A panels and B panels in L2.
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  int bm, bn;
  {
    const int pid = blockIdx.x;
    constexpr int GM = 8;
    const int group = pid / (GM * nbn);
    const int first = group * GM;
    const int gsz = min(nbm - first, GM);
    const int in = pid - group * GM * nbn;
    bm = first + in % gsz;
    bn = in / gsz;
  }
  const int m0 = bm * BM, n0 = bn * BN;

  // B row segment holding this column block (segments are multiples of BN except the last).
  const bf16* Bseg;
  int nb0, nrows;
  if (n0 < g.nseg0) { Bseg = (const bf16*)g.B0; nb0 = n0; nrows = g.nseg0; }
  else if (n0 < g.nseg0 + g.nseg1) { Bseg = (const bf16*)g.B1; nb0 = n0 - g.nseg0; nrows = g.nseg1; }
  else { Bseg = (const bf16*)g.B2; nb0 = n0 - g.nseg0 - g.nseg1; nrows = N - g.nseg0 - g.nseg1; }

  const bf16* const A = (const bf16*)g.A;
  const int lda = g.lda, ldb = g.ldb;

  u32x4 ra[AC], rb[BC];
  const bf16* pa[AC];
  const bf16* pb[BC];
  int la[AC], lb[BC];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = c & 7;
    pa[i] = A + (size_t)min(m0 + r, M - 1) * lda + kc * 8;
    la[i] = r * BK + ((kc ^ swz8(r)) << 3);
  }
#pragma unroll
  for (int i = 0; i < BC; ++i) {
    const int c = tid + i * NT, r = c >> 3, kc = c & 7;
    pb[i] = Bseg + (size_t)min(nb0 + r, nrows - 1) * ldb + kc * 8;
    lb[i] = r * BK + ((kc ^ swz8(r)) << 3);
  }
#define GEMM_GLOAD(k0)                                                      \
  do {                                                                      \
    _Pragma("unroll") for (int i = 0; i < AC; ++i) ra[i] = *(const u32x4*)(pa[i] + (k0)); \
    _Pragma("unroll") for (int i = 0; i < BC; ++i) rb[i] = *(const u32x4*)(pb[i] + (k0)); \
  } while (0)
#define GEMM_SSTORE(buf)                                                                        \
  do {                                                                                          \
    _Pragma("unroll") for (int i = 0; i < AC; ++i) *(u32x4*)(As + (buf) * BM * BK + la[i]) = ra[i]; \
    _Pragma("unroll") for (int i = 0; i < BC; ++i) *(u32x4*)(Bs + (buf) * BN * BK + lb[i]) = rb[i]; \
  } while (0)

  // Fragment read offsets (elements) for k-substep 0; substep kk adds chunk 2*kk.
  int oa[FM], ob[FN];
  const int hl = lane >> 5, rl = lane & 31;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) oa[fm] = (wm * TM + fm * 32 + rl) * BK;
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) ob[fn] = (wn * TN + fn * 32 + rl) * BK;
  const int sa = swz8(rl);  // rows differ from rl by multiples of 32: same swizzle

  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.f;

  const int nk = K / BK;
  GEMM_GLOAD(0);
  GEMM_SSTORE(0);
  if (nk > 1) GEMM_GLOAD(BK);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bf16* Ab = As + buf * BM * BK;
    const bf16* Bb = Bs + buf * BN * BK;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int co = ((2 * kk + hl) ^ sa) << 3;
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) af[fm] = *(const bf16x8*)(Ab + oa[fm] + co);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) bfr[fn] = *(const bf16x8*)(Bb + ob[fn] + co);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
    }
    if (kt + 1 < nk) GEMM_SSTORE(buf ^ 1);
    if (kt + 2 < nk) GEMM_GLOAD((kt + 2) * BK);
    __syncthreads();
  }

#undef GEMM_GLOAD
#undef GEMM_SSTORE

  // ---------------------------------------------------------------- epilogues
  // acc[fm][fn][r] is C[row][col] with row = m0 + wm*TM + fm*32 + 8*(r/4) + 4*hl + r%4 and
  // col = n0 + wn*TN + fn*32 + rl.
  const int rbase = m0 + wm * TM + 4 * hl;
  const int cbase = n0 + wn * TN + rl;

  if constexpr (EPI == EPI_STORE || EPI == EPI_RELU2) {
    bf16* out = (bf16*)g.out;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = cbase + fn * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + fm * 32 + 8 * (r >> 2) + (r & 3);
          float v = acc[fm][fn][r];
          if (EPI == EPI_RELU2) { v = fmaxf(v, 0.f); v = v * v; }
          if (row < M && col < N) out[(size_t)row * g.ldo + col] = (bf16)v;
        }
      }
  } else if constexpr (EPI == EPI_RESID) {
    float* out = (float*)g.out;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = cbase + fn * 32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = rbase + fm * 32 + 8 * (r >> 2) + (r & 3);
          if (row < M && col < N) {
            float* p = out + (size_t)row * g.ldo + col;
            *p = *p + acc[fm][fn][r];
          }
        }
      }
  } else if constexpr (EPI == EPI_QKV) {
    bf16* qk = (bf16*)g.out;
    bf16* vt = (bf16*)g.vt;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = cbase + fn * 32;
      if (col >= N) continue;
      if (col < g.nqk) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rbase + fm * 32 + 8 * (r >> 2) + (r & 3);
            if (row < M) qk[(size_t)row * g.ldo + col] = (bf16)acc[fm][fn][r];
          }
      } else {
        const int vc = col - g.nqk, gg = vc / g.D, d = vc - gg * g.D;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = rbase + fm * 32 + 8 * j;  // rows row..row+3 share one sequence (T % 4 == 0)
            if (row < M) {
              const int b = row / g.T, t = row - b * g.T;
              bf16x4 v4;
#pragma unroll
              for (int i = 0; i < 4; ++i) v4[i] = (bf16)acc[fm][fn][4 * j + i];
              *(bf16x4*)(vt + ((size_t)(b * g.Hkv + gg) * g.D + d) * g.T + t) = v4;
            }
          }
      }
    }
  } else if constexpr (EPI == EPI_CE) {
    // Per-row partial sums over this block's columns, reduced through LDS (free after the
    // main loop's final barrier).
    constexpr int RW = WN * 32 + 1;  // padded row stride of the reduction buffer
    static_assert(BM * RW * 4 <= 2 * (BM + BN) * BK * 2, "reduction buffer exceeds LDS");
    float* red = (float*)lds;
    const float cap = g.cap;
    const float k1 = 2.0f / cap * GPT_LOG2E, k2 = -2.0f * cap * GPT_LOG2E;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rloc = wm * TM + fm * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const int row = m0 + rloc;
        const int y = (g.targets != nullptr && row < M) ? g.targets[row] : -1;
        float s = 0.f;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = cbase + fn * 32;
          const float z = acc[fm][fn][r];
          if (col < N) {
            s += ce_term(z, k1, k2);
            // raw logits: the loss kernel and the logits pass apply the softcap
            if (col == y) g.tgt_logit[row] = z;
            if (g.logits != nullptr && row < M) g.logits[(size_t)row * N + col] = z;
          }
        }
        red[rloc * RW + wn * 32 + rl] = s;
      }
    __syncthreads();
    for (int rloc = tid; rloc < BM; rloc += NT) {
      const int row = m0 + rloc;
      if (row < M) {
        float s = 0.f;
        for (int j = 0; j < WN * 32; ++j) s += red[rloc * RW + j];
        g.partial[(size_t)row * g.nnb + bn] = s;
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t run_bf16(Epi epi, const GemmArgs& a, hipStream_t s) {
  const int grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int NT = WM * WN * 64;
  switch (epi) {
    case EPI_STORE: gemm_bf16_kernel<BM, BN, WM, WN, EPI_STORE><<<grid, NT, 0, s>>>(a); break;
    case EPI_RELU2: gemm_bf16_kernel<BM, BN, WM, WN, EPI_RELU2><<<grid, NT, 0, s>>>(a); break;
    case EPI_RESID: gemm_bf16_kernel<BM, BN, WM, WN, EPI_RESID><<<grid, NT, 0, s>>>(a); break;
    case EPI_QKV: gemm_bf16_kernel<BM, BN, WM, WN, EPI_QKV><<<grid, NT, 0, s>>>(a); break;
    case EPI_CE: gemm_bf16_kernel<BM, BN, WM, WN, EPI_CE><<<grid, NT, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ fp32 path
// 64x64 tiles, 256 threads each computing 4x4 outputs; A and B tiles transposed into LDS.
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[FK][FT + 4];
  __shared__ float Bs[FK][FT + 4];
  __shared__ float red[FT][17];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int nbn = (g.N + FT - 1) / FT;
  const int bm = blockIdx.x / nbn, bn = blockIdx.x % nbn;
  const int m0 = bm * FT, n0 = bn * FT;
  const float* A = (const float*)g.A;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += FK) {
    for (int e = tid; e < FT * FK; e += 256) {
      const int r = e / FK, c = e % FK;
      const int row = m0 + r, k = k0 + c;
      As[c][r] = (row < g.M && k < g.K) ? A[(size_t)row * g.lda + k] : 0.f;
      const int n = n0 + r;
      float bv = 0.f;
      if (n < g.N && k < g.K) {
        const float* Bp;
        int nn;
        if (n < g.nseg0) { Bp = (const float*)g.B0; nn = n; }
        else if (n < g.nseg0 + g.nseg1) { Bp = (const float*)g.B1; nn = n - g.nseg0; }
        else { Bp = (const float*)g.B2; nn = n - g.nseg0 - g.nseg1; }
        bv = Bp[(size_t)nn * g.ldb + k];
      }
      Bs[c][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < FK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { av[i] = As[k][ty * 4 + i]; bv[i] = Bs[k][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  if constexpr (EPI == EPI_CE) {
    const float cap = g.cap;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + ty * 4 + i;
      const int y = (g.targets != nullptr && row < g.M) ? g.targets[row] : -1;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + tx * 4 + j;
        if (row < g.M && col < g.N) {
          const float zh = cap * tanhf(acc[i][j] / cap);
          s += expf(zh - cap);
          if (col == y) g.tgt_logit[row] = acc[i][j];
          if (g.logits != nullptr) g.logits[(size_t)row * g.N + col] = acc[i][j];
        }
      }
      red[ty * 4 + i][tx] = s;
    }
    __syncthreads();
    if (tid < FT) {
      const int row = m0 + tid;
      if (row < g.M) {
        float s = 0.f;
        for (int j = 0; j < 16; ++j) s += red[tid][j];
        g.partial[(size_t)row * g.nnb + bn] = s;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
        if (row >= g.M || col >= g.N) continue;
        float v = acc[i][j];
        float* out = (float*)g.out + (size_t)row * g.ldo + col;
        if (EPI == EPI_RELU2) { v = fmaxf(v, 0.f); v = v * v; }
        if (EPI == EPI_RESID) *out = *out + v;
        else *out = v;
      }
  }
}

}  // namespace

int gemm_bf16_ce_blocks(int N) { return (N + 127) / 128; }
int gemm_f32_ce_blocks(int N) { return (N + FT - 1) / FT; }

hipError_t launch_gemm_bf16(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % BK || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
  if (epi == EPI_CE) return run_bf16<256, 128, 2, 2>(epi, a, s);  // must match gemm_bf16_ce_blocks
  // Interior column-segment boundaries must fall on block-column boundaries.
  auto seg_ok = [&](int bn) {
    const int e0 = a.nseg0, e1 = a.nseg0 + a.nseg1;
    return (e0 >= a.N || e0 % bn == 0) && (e1 >= a.N || e1 % bn == 0);
  };
  const bool n256 = seg_ok(256), n128 = seg_ok(128);
  const long tiles256 = (long)((a.M + 255) / 256) * ((a.N + 255) / 256);
  if (n256 && tiles256 >= 1024) return run_bf16<256, 256, 2, 2>(epi, a, s);
  if (n128) return run_bf16<256, 128, 2, 2>(epi, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_f32(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipErrorInvalidValue;
  const int grid = ((a.M + FT - 1) / FT) * ((a.N + FT - 1) / FT);
  switch (epi) {
    case EPI_STORE: case EPI_QKV: gemm_f32_kernel<EPI_STORE><<<grid, 256, 0, s>>>(a); break;
    case EPI_RELU2: gemm_f32_kernel<EPI_RELU2><<<grid, 256, 0, s>>>(a); break;
    case EPI_RESID: gemm_f32_kernel<EPI_RESID><<<grid, 256, 0, s>>>(a); break;
    case EPI_CE: gemm_f32_kernel<EPI_CE><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gptk
