// Causal sliding-window attention, flash style (online softmax, no T x T matrix in memory).
//
// Source: "The Mathematics of Karpathy's nanochat", section "Scaled Dot-Product Attention with
// Sliding Window": query i sees key j iff j <= i and i - j < w; softmax over the visible keys;
// output = weighted sum of values.  q and k arrive already rotated (RoPE) and normalised
// (QK-norm); the logit is scale * <q, k>.
//
// bf16 kernel (gfx950, head_dim 128 or 64).  A block owns 256 queries of one (batch, head)
// and eight wavefronts (two per SIMD), 32 queries each; only key tiles (64 keys) that
// intersect the block's window band are visited.  Each wavefront computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 so that every lane holds one query's logits (query = lane % 32):
// the softmax max needs one exchange with lane ^ 32 and the running sum none.  K rows are
// stored in LDS with bits 2 and 3 of the key index swapped, which makes each lane's S^T
// accumulators hold 8 consecutive keys per 16-key step; packed to bf16 they are directly the
// B operand of O^T += V^T P^T, whose A operand is read from the transposed value tile
// [D][64 keys].  Values arrive transposed ([B][Hkv][D][T]) from the QKV projection's epilogue.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gptk {
namespace {

constexpr int BKV = 64;

// s_waitcnt immediate: at most n vector-memory operations outstanding (gfx9 encoding).
constexpr int vmcnt_le(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ int swap23(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}
// 16-byte chunk swizzles: K tile rows have D/8 chunks, V^T tile rows have 8.
template <int D> __device__ __forceinline__ int swzk(int r) { return (D == 128) ? (r & 15) : (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swzv(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 256 queries per block, 8 wavefronts (two per SIMD, so one wavefront's softmax VALU work
// overlaps the other's MFMAs), K and V^T tiles streamed global -> LDS with
// buffer_load ... lds into a 3-stage ring, the logit scale folded into one FMA before exp2, and
// lazy rescaling: a row's reference maximum moves only when a new logit exceeds it by more than
// 2^8 (in log2 units).  Numerator and denominator share the reference, so the result is exact;
// the bound keeps every probability <= 256.
//
// PRIOR (looped trunk, "looped-nanochat-d24", section "What is the routing loop?"): the logits
// also carry g * <q1, k1> from pass 1's q and k of this layer (qk1, the qk layout), g =
// softplus(gate_logit[layer]).  This is attention over the augmented width [q, g q1] . [k, k1]:
// K tiles hold both halves (k from qk, k1 from qk1), the query fragments both (q1 scaled by g
// before rounding), so S^T takes 2 D/16 k-steps; V and everything after are unchanged.  This
// form also runs 8 wavefronts (two per SIMD; the doubled query fragments bring it to 254 VGPRs)
// and a 3-stage ring of 48 KB stages.
constexpr int STG = 3;

template <int D, int NW, bool PRIOR, bool BOUNDED>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(const bf16* __restrict__ qk,
                                                                const bf16* __restrict__ vt,
                                                                bf16* __restrict__ o, int B, int T,
                                                                int H, int Hkv, int window, float c,
                                                                const bf16* __restrict__ qk1,
                                                                const float* __restrict__ gate_logit,
                                                                int layer) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BQ2 = NW * 32;          // queries per block
  constexpr int NK = PRIOR ? 2 : 1;     // K halves (k, k1)
  constexpr int KCH = D / 8;            // 16-byte chunks per K row
  constexpr int DT = D / 32;            // 32-row tiles of O^T
  constexpr int KS = D / 16;            // k-steps of S^T per K half
  constexpr int KROWS = 64 / KCH;       // K rows per 1 KB DMA instruction
  constexpr int KI = BKV * KCH / 64 / NW, VI = D * 8 / 64 / NW;  // DMA instructions per wave
  static_assert(KI * NW * 64 == BKV * KCH && VI * NW * 64 == D * 8, "DMA tiling");
  __shared__ __attribute__((aligned(16))) bf16 Ks[STG][NK * BKV * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[STG][D * BKV];

  // Blocks are dispatched in launch order, so the linear block index runs over query tiles
  // from the last (the most key tiles) to the first, every (head, batch) pair within a tile
  // row: the longest blocks start first and the short ones fill in at the end.
  const int nqt = (T + BQ2 - 1) / BQ2;
  const int hb = (int)blockIdx.x % (H * B), qrank = (int)blockIdx.x / (H * B);
  const int qt = nqt - 1 - qrank;
  const int h = hb % H, b = hb / H;
  const int g = (h * Hkv) / H;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int hl = lane >> 5, rl = lane & 31;
  const int ldqk = (H + Hkv) * D;
  const int qb = qt * BQ2;
  const int qw = qb + wid * 32;
  const int myq = qw + rl;

  bf16x8 qf[NK * KS];
  {
    const size_t qrow = (size_t)(b * T + min(myq, T - 1)) * ldqk + h * D + 8 * hl;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8*)(qk + qrow + 16 * s);
    if constexpr (PRIOR) {
      const float z = gate_logit[layer];
      const float gp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));  // softplus
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 u = *(const bf16x8*)(qk1 + qrow + 16 * s);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[KS + s][e] = (bf16)((float)u[e] * gp);
      }
    }
  }

  const int kmin = max(0, qb - window + 1);
  const int kmax = min(T - 1, qb + BQ2 - 1);
  const int t0 = kmin / BKV, t1 = kmax / BKV;

  // DMA sources.  K: buffer over this sequence's rows of the qk matrix, soffset = tile start.
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qk + (size_t)b * T * ldqk + (H + g) * D), (short)0, (int)min((size_t)T * ldqk * 2, (size_t)0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vt + (size_t)(b * Hkv + g) * D * T), (short)0, (int)min((size_t)D * T * 2, (size_t)0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t rk1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((PRIOR ? qk1 : qk) + (size_t)b * T * ldqk + (H + g) * D), (short)0, (int)min((size_t)T * ldqk * 2, (size_t)0x7fffffff), 0x00020000);
  int ko[KI], vo[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int pr = KROWS * (wid * KI + i) + lane / KCH, slot = lane % KCH;
    ko[i] = (swap23(pr) * ldqk + ((slot ^ swzk<D>(pr)) << 3)) * 2;
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int d = 8 * (wid * VI + i) + (lane >> 3), slot = lane & 7;
    vo[i] = (d * T + ((slot ^ swzv(d)) << 3)) * 2;
  }
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  auto issue = [&](int t) {
    const int st = (t - t0) % STG, j0 = t * BKV;
#pragma unroll
    for (int i = 0; i < KI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(&Ks[st][(wid * KI + i) * 512]), 16, ko[i], j0 * ldqk * 2, 0, 0);
    if constexpr (PRIOR) {
#pragma unroll
      for (int i = 0; i < KI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk1, (lds_ptr_t)(&Ks[st][BKV * D + (wid * KI + i) * 512]), 16, ko[i], j0 * ldqk * 2, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(&Vs[st][(wid * VI + i) * 512]), 16, vo[i], j0 * 2, 0, 0);
  };

  f32x16 ot[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) ot[d][r] = 0.f;
  float m_ref = -1e30f, l_run = 0.f;  // reference max in log2 units (finite: keeps -inf logits at p = 0)

  auto active_tile = [&](int t) {
    const int j0 = t * BKV;
    return (j0 <= qw + 31) && (j0 + BKV - 1 >= qw - window + 1) && (qw < T);
  };
  // S^T = K Q^T for one tile: sv[rt][r] is the raw logit of key
  // j0 + rt*32 + 16*(r>>3) + 8*hl + 4*((r>>2)&1) + (r&3) for query myq.
  auto scores = [&](int t, f32x16 (&sv)[2]) {
    const int st = (t - t0) % STG;
    const bf16* kp[2];
    int sw[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int kr = rt * 32 + rl;
      kp[rt] = &Ks[st][kr * D];
      sw[rt] = swzk<D>(kr);
    }
    // k-step outer, row tile inner: consecutive MFMAs never chain on one accumulator; the
    // first k-step takes a zero accumulator (an inline constant, no register zeroing)
    const f32x16 zero = {};
#pragma unroll
    for (int s2 = 0; s2 < NK * KS; ++s2)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int half = s2 / KS, ss = s2 % KS;  // K half (k or k1) and k-step within it
        const bf16x8 a = *(const bf16x8*)(kp[rt] + half * BKV * D + (((2 * ss + hl) ^ sw[rt]) << 3));
        sv[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s2], s2 == 0 ? zero : sv[rt], 0, 0, 0);
      }
  };

  // Software pipeline: the logits of tile t+1 are issued to the matrix cores before the softmax
  // of tile t runs on the VALU, then tile t's P V^T follows.  Ring stages hold tiles t, t+1 and
  // t+2; the barrier at the top of iteration t publishes tile t+1 and retires tile t-1's stage.
  f32x16 sA[2], sB[2];
  issue(t0);
  if (t0 + 1 <= t1) issue(t0 + 1);
  if (t0 + 1 <= t1) __builtin_amdgcn_s_waitcnt(vmcnt_le(NK * KI + VI));
  else __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
  __syncthreads();
  bool act_cur = active_tile(t0);
  if (act_cur) scores(t0, sA);
  const bf16x2 ones2 = {(bf16)1.0f, (bf16)1.0f};
  // One pipeline step: tile t's softmax and P V^T with tile t+1's logits issued first.  Called
  // with the two logit register sets in alternating roles (loop unrolled by two: no copies).
  auto step = [&](int t, f32x16 (&scur)[2], f32x16 (&snxt)[2]) {
      const int st = (t - t0) % STG;
      const int j0 = t * BKV;
      const bool more = t + 1 <= t1;
      if (more) {
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));  // own loads of tile t+1 landed
        __syncthreads();                          // everyone's; stage of tile t-1 is free
        if (t + 2 <= t1) issue(t + 2);
      }
      const bool act_nxt = more && active_tile(t + 1);
      if (act_nxt) scores(t + 1, snxt);
      if (act_cur) {
        const bool full = (j0 + BKV - 1 <= qw) && (qw + 31 - j0 < window);
        if (!full) {
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = j0 + rt * 32 + 16 * (r >> 3) + 8 * hl + 4 * ((r >> 2) & 1) + (r & 3);
              if (key > myq || myq - key >= window) scur[rt][r] = -INFINITY;
            }
        }
        bf16x8 pf[4];
        if constexpr (BOUNDED) {
          // reference 0 (see attn_launch_bounded): p = 2^(s c); the row sum adds the rounded
          // probabilities that P V^T uses, two at a time
          float ps[2] = {0.f, 0.f};
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              bf16x2 pp;
              pp[0] = (bf16)exp2_fast(scur[rt][r] * c);
              pp[1] = (bf16)exp2_fast(scur[rt][r + 1] * c);
              pf[rt * 2 + (r >> 3)][r & 7] = pp[0];
              pf[rt * 2 + (r >> 3)][(r & 7) + 1] = pp[1];
              ps[rt] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, ps[rt], false);
            }
          l_run += ps[0] + ps[1];
        } else {
          float mt[16];  // tree reduction: depth 5 instead of a 32-long chain
#pragma unroll
          for (int r = 0; r < 16; ++r) mt[r] = fmaxf(scur[0][r], scur[1][r]);
#pragma unroll
          for (int w = 8; w > 0; w >>= 1)
#pragma unroll
            for (int r = 0; r < w; ++r) mt[r] = fmaxf(mt[r], mt[r + w]);
          float mx = fmaxf(mt[0], __shfl_xor(mt[0], 32, 64)) * c;
          const bool grow = mx > m_ref + 8.0f;
          if (__builtin_amdgcn_ballot_w64(grow)) {
            const float corr = grow ? exp2_fast(m_ref - mx) : 1.0f;
            if (grow) m_ref = mx;
            l_run *= corr;
#pragma unroll
            for (int d = 0; d < DT; ++d)
#pragma unroll
              for (int r = 0; r < 16; ++r) ot[d][r] *= corr;
          }
          const float nm = -m_ref;
          float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums instead of one chain
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = exp2_fast(fmaf(scur[rt][r], c, nm));
              ps[r & 3] += p;
              pf[rt * 2 + (r >> 3)][r & 7] = (bf16)p;
            }
          l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        }
        // k-step outer, d tile inner: DT independent accumulators between dependent MFMAs
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int d = 0; d < DT; ++d) {
            const int vr = d * 32 + rl;
            const bf16x8 a = *(const bf16x8*)(&Vs[st][vr * BKV] + (((2 * s2 + hl) ^ swzv(vr)) << 3));
            ot[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s2], ot[d], 0, 0, 0);
          }
      }
      act_cur = act_nxt;
  };
  for (int t = t0; t <= t1; t += 2) {
    step(t, sA, sB);
    if (t + 1 <= t1) step(t + 1, sB, sA);
  }

  const float l = l_run + __shfl_xor(l_run, 32, 64);
  // head_dim 128 without the prior: the wavefront's 32 output rows go out through LDS (the K/V
  // ring, free once every wavefront is past its last tile) as whole rows, 16 bytes per lane with
  // consecutive lanes on consecutive chunks of a row, instead of 8-byte pieces of 32 rows per
  // store (d24: 117.2 -> 114.2 us per launch).  The head_dim-64 and prior forms store directly
  // (staged, they measured level and 2 % slower).
  constexpr bool STAGE_O = D == 128 && !PRIOR;
  if constexpr (STAGE_O) {
    constexpr int OP = D + 8;                                 // staging pitch (bf16), 16-byte rows
    constexpr int WB = 32 * OP;                               // staging elements per wavefront
    constexpr int KW = (int)(sizeof(Ks) / sizeof(bf16)) / WB; // wavefronts staged in Ks, the rest in Vs
    static_assert(KW + (int)(sizeof(Vs) / sizeof(bf16)) / WB >= NW, "output staging exceeds the K/V ring");
    __syncthreads();  // every wavefront is done with the ring
    bf16* const stg = wid < KW ? &Ks[0][0] + wid * WB : &Vs[0][0] + (wid - KW) * WB;
    {
      const float inv = 1.0f / l;  // rows past T (inf here) are not stored
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 v4;
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = (bf16)(ot[d][4 * j + i] * inv);
          *(bf16x4*)(stg + rl * OP + d * 32 + 8 * j + 4 * hl) = v4;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int OCH = D / 8;  // 16-byte chunks per output row
#pragma unroll
    for (int k = 0; k < 32 * OCH / 64; ++k) {
      const int idx = lane + 64 * k, r = idx / OCH, ch = idx % OCH;
      const int q = qw + r;
      if (q < T)
        *(bf16x8*)(o + (size_t)(b * T + q) * (H * D) + h * D + 8 * ch) = *(const bf16x8*)(stg + r * OP + 8 * ch);
    }
  } else if (myq < T) {
    const float inv = 1.0f / l;
    bf16* op = o + (size_t)(b * T + myq) * (H * D) + h * D;
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = (bf16)(ot[d][4 * j + i] * inv);
        *(bf16x4*)(op + d * 32 + 8 * j + 4 * hl) = v4;
      }
  }
#endif
}

// fp32 path: one thread per query, keys read from global memory.  With qkv1 (looped pass 2)
// each logit adds g * <q1_i, k1_j> from pass 1's q and k (same layout as qkv).
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ qkv, float* __restrict__ o,
                                                      int T, int H, int Hkv, int window, float scale,
                                                      const float* __restrict__ qkv1,
                                                      const float* __restrict__ gate_logit, int layer) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= T) return;
  const int g = (h * Hkv) / H;
  const int ld = (H + 2 * Hkv) * D;
  const float* q = qkv + (size_t)(b * T + i) * ld + h * D;
  float qv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { qv[d] = q[d]; acc[d] = 0.f; }
  float gp = 0.f;
  if (qkv1 != nullptr) {
    const float z = gate_logit[layer];
    gp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));  // softplus
  }
  float m = -INFINITY, l = 0.f;
  const int j_lo = max(0, i - window + 1);
  for (int j = j_lo; j <= i; ++j) {
    const float* k = qkv + (size_t)(b * T + j) * ld + (H + g) * D;
    const float* v = qkv + (size_t)(b * T + j) * ld + (H + Hkv + g) * D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], k[d], s);
    if (qkv1 != nullptr) {
      const float* q1 = qkv1 + (size_t)(b * T + i) * ld + h * D;
      const float* k1 = qkv1 + (size_t)(b * T + j) * ld + (H + g) * D;
      float s1 = 0.f;
      for (int d = 0; d < D; ++d) s1 = fmaf(q1[d], k1[d], s1);
      s = fmaf(gp, s1, s);
    }
    s *= scale;
    const float m_new = fmaxf(m, s);
    const float corr = expf(m - m_new);
    const float p = expf(s - m_new);
    l = l * corr + p;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * corr + p * v[d];
    m = m_new;
  }
  float* op = o + (size_t)(b * T + i) * (H * D) + h * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
}

}  // namespace

// Whether the attention kernel may take 0 as every query's softmax reference.  q and k arrive
// RMS-normalised per head (|q|^2, |k|^2 <= D before bf16 rounding, which adds at most a factor
// (1 + 2^-8) to each norm), so every logit in log2 units lies within +-scale * D * log2(e) * 1.008.
// Within +-32 the exponentials lie in [2^-32, 2^32]: no fp32 overflow or underflow, also summed
// over 2^20 keys, and softmax does not depend on the reference.  The nanochat scale 1/sqrt(D)
// gives 16.4 (D = 128) and 11.6 (D = 64).
bool attn_launch_bounded(float scale, int D) {
  return (double)scale * D * 1.4426950408889634 * 1.01 <= 32.0;
}

hipError_t launch_attn_bf16(const void* qk, const void* vt, void* o, int B, int T, int H, int Hkv,
                            int D, int window, float scale, hipStream_t s, const void* qk1,
                            const float* gate_logit, int layer) {
  if (T % BKV) return hipErrorInvalidValue;
  const float sl2 = scale * GPT_LOG2E;
  const bf16* q = (const bf16*)qk;
  const bf16* v = (const bf16*)vt;
  bf16* out = (bf16*)o;
  // Logits of normalised q and k lie within +-scale * D (in log2 units, times log2 e); with the
  // looped prior within +-scale * D * (1 + g).
  if (qk1 != nullptr) {  // looped pass 2: prior from pass 1
    if (D != 128 || gate_logit == nullptr) return hipErrorInvalidValue;
    const dim3 grid(((T + 255) / 256) * H * B);
    GPTK_LAUNCH((attn_bf16_kernel<128, 8, true, false>), grid, 512, s, q, v, out, B, T, H, Hkv, window, sl2,
                (const bf16*)qk1, gate_logit, layer);
    return hipGetLastError();
  }
  const dim3 grid(((T + 255) / 256) * H * B);
  const bool bounded = attn_launch_bounded(scale, D);
  if (D == 128) {
    if (bounded)
      GPTK_LAUNCH((attn_bf16_kernel<128, 8, false, true>), grid, 512, s, q, v, out, B, T, H, Hkv, window, sl2,
                  (const bf16*)nullptr, (const float*)nullptr, 0);
    else
      GPTK_LAUNCH((attn_bf16_kernel<128, 8, false, false>), grid, 512, s, q, v, out, B, T, H, Hkv, window, sl2,
                  (const bf16*)nullptr, (const float*)nullptr, 0);
  } else if (D == 64) {
    if (bounded)
      GPTK_LAUNCH((attn_bf16_kernel<64, 8, false, true>), grid, 512, s, q, v, out, B, T, H, Hkv, window, sl2,
                  (const bf16*)nullptr, (const float*)nullptr, 0);
    else
      GPTK_LAUNCH((attn_bf16_kernel<64, 8, false, false>), grid, 512, s, q, v, out, B, T, H, Hkv, window, sl2,
                  (const bf16*)nullptr, (const float*)nullptr, 0);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn_f32(const float* qkv, float* o, int B, int T, int H, int Hkv, int D,
                           int window, float scale, hipStream_t s, const float* qkv1,
                           const float* gate_logit, int layer) {
  if (qkv1 != nullptr && gate_logit == nullptr) return hipErrorInvalidValue;
  const dim3 grid((T + 63) / 64, H, B);
  if (D == 128) GPTK_LAUNCH(attn_f32_kernel<128>, grid, 64, s, qkv, o, T, H, Hkv, window, scale, qkv1, gate_logit, layer);
  else if (D == 64) GPTK_LAUNCH(attn_f32_kernel<64>, grid, 64, s, qkv, o, T, H, Hkv, window, scale, qkv1, gate_logit, layer);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gptk
