// Decode-step kernels: one new token per row against a KV cache, and sampling of the next token.
//
// Sources: "The Mathematics of Karpathy's nanochat", section "Inference: Generating Text" (the
// autoregressive loop: logits at the last position, then a draw) and its "Sampling Controls"
// (temperature, top-k filtering, greedy at temperature 0).  A step at position t computes what
// the full forward computes at position t -- attention is causal, so the keys and values of
// positions < t are those cached by earlier steps ("Scaled Dot-Product Attention with Sliding
// Window": query t sees keys j <= t with t - j < w).
//
// With B rows the weight products are [B, K] x [N, K]^T: every weight is read once per step and
// used B times, so they stream at HBM speed.  Even so, the products run on MFMA: at B = 8 a VALU
// product needs 8 multiply-adds per 2-byte weight, more than the vector units retire at HBM rate.
#include "common.h"
#include "kernels.h"

namespace gptk {
namespace {

constexpr int GV_ROWS = 32;   // weight rows per block (one 32x32 MFMA output tile, batch in N)
constexpr int GV_WAVES = 4;   // wavefronts per block for short K ranges (8 for longer ones)
constexpr int GV_KB = 64;     // K per wavefront step: four 32x32x16 MFMAs
constexpr int GV_TARGET_BLOCKS = 2048;  // K splits aim at this many blocks (2048: 0.6 % faster d24 step than 1024)

// Per-(row b, column n) epilogue of a decode-step product.
struct GvEpi {
  int kind;           // DEC_* below
  void* out; int ldo; // STORE: f32; RELU2: activation type; RESID, RESID_RS: f32 (x += v); LOGITS: f32
  float cap;
  const int32_t* pos; const int32_t* tokens; int T; int V;  // LOGITS: rows with bad input -> NaN
  const float* rs; int rs_n; float eps;  // row scale: 1/rms of row b from rs[b * rs_n + j], j < rs_n
  bf16* xb; float* ss;                   // RESID_RS: bf16(x) [B][ldo] and ss[b * gridDim.x + block]
};

template <typename AT>
__device__ __forceinline__ void gv_apply(const GvEpi& e, int b, int n, float v) {
  const size_t o = (size_t)b * e.ldo + n;
  switch (e.kind) {
    case DEC_STORE: ((float*)e.out)[o] = v; break;
    case DEC_RELU2: { const float r = fmaxf(v, 0.f); ((AT*)e.out)[o] = from_f32<AT>(r * r); } break;
    case DEC_RESID: ((float*)e.out)[o] += v; break;
    case DEC_LOGITS: {
      bool bad = false;
      if (e.pos != nullptr) {
        const int p = e.pos[b], t = e.tokens[b];
        bad = p < 0 || p >= e.T || t < 0 || t >= e.V;
      }
      ((float*)e.out)[o] = bad ? __builtin_nanf("") : e.cap * tanhf(v / e.cap);
    } break;
  }
}

// bf16 weights and activations: y[b][n] = sum_k act[b][k] W[n][k] for b < B <= 32.  A block
// owns 32 weight rows (three row segments W0 | W1 | W2 with boundaries on multiples of 32) and
// one of KS contiguous ranges of 64-column K steps; its NW wavefronts take the range's steps in
// turn.  In a step, lane l (row l % 32, half g = l / 32) holds W[row][kb + 32g + 8m .. +8] for
// MFMA m = 0..3 and the batch operand holds act[b = l % 32][the same columns], so each MFMA sums
// 16 columns and the four cover the step.  The weight tiles (32 rows x 64 columns, 4 KB) do not
// go to registers directly: loaded that way, each 16-byte-per-lane load touches 32 rows, i.e. 32
// cache lines with 32 bytes used of each.  Instead each wavefront copies its steps' tiles into
// its own LDS slots by DMA (buffer_load ... lds), 8 rows x 128 bytes per instruction with the
// 16-byte chunks of row r at slot c ^ swz8(r), issues up to DEPTH steps' copies (and the batch
// operand's loads) at once, waits for them, and reads the fragments from LDS.  The wavefronts'
// tiles are summed through LDS in a fixed order.  With KS > 1 the block stores its tile as
// partial[ks][b][n] and the consumer of the product sums the KS tiles in split order (no block
// waits on another); with KS = 1 the epilogue is applied here.
// Row scale (e.rs given): the batch operand is bf16(x) of an un-normalised residual stream x and
// the outputs of row b (partial tiles included) are scaled by 1/rms_b = (sum / K + eps)^-1/2,
// sum = the producer's per-block sums of squares of row b's fp32 values, added in block order:
// the row scale the forward's GEMMs apply to an un-normalised input.
// DEC_RESID_RS (KS = 1): x += y, and the block also writes bf16(x) for the next product and the
// sum of squares of its 32 columns of each row of x (columns in order), ss[b * nblocks + block].
__device__ __forceinline__ int gv_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// s_waitcnt immediate for vmcnt = 0 (gfx9 encoding; expcnt and lgkmcnt at their maxima)
constexpr int GV_VMCNT0 = 0x0F70;
typedef __attribute__((address_space(3))) void* gv_lds_t;
template <int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) void gemv_bf16_kernel(
    const bf16* __restrict__ act, int lda, int B, const bf16* __restrict__ W0,
    const bf16* __restrict__ W1, const bf16* __restrict__ W2, int nseg0, int nseg1, int N, int K,
    int KS, float* __restrict__ partial, GvEpi e) {
  __shared__ __attribute__((aligned(16))) bf16 wl[NW][DEPTH][GV_ROWS * GV_KB];
  __shared__ float rsc[32];                 // row scales (e.rs)
  __shared__ float sq[32][GV_ROWS + 1];     // DEC_RESID_RS: squares of the updated x
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wids = __builtin_amdgcn_readfirstlane(wid);
  const int rb = blockIdx.x / KS, ks = blockIdx.x % KS;
  const int n0 = rb * GV_ROWS;
  const bf16* W;
  int r0;
  if (n0 < nseg0) { W = W0; r0 = n0; }
  else if (n0 < nseg0 + nseg1) { W = W1; r0 = n0 - nseg0; }
  else { W = W2; r0 = n0 - nseg0 - nseg1; }
  const int row = lane & 31, g = lane >> 5;
  const bool b_ok = row < B;  // the batch operand's lane row is b
  const bf16* ap = act + (size_t)row * lda + 32 * g;
  const int nks = K / GV_KB, s0 = (int)((long)ks * nks / KS), s1 = (int)((long)(ks + 1) * nks / KS);
  // The block's rows as a buffer resource: rows past N (last block) read as zero.  DMA lane L of
  // instruction i fetches row 8i + L/8, chunk (L % 8) ^ swz(row); the K offset rides in soffset.
  const int nrow = N - n0 < GV_ROWS ? N - n0 : GV_ROWS;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (size_t)r0 * K), (short)0, nrow * K * 2, 0x00020000);
  int voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (lane >> 3) + 8 * i;
    voff[i] = rr * K * 2 + (((lane & 7) ^ gv_swz(rr)) << 4);
  }
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const bf16x8 zero = {};
  const int sw = gv_swz(row);
  // Row scales: wavefront w sums the per-block sums of squares of rows w, w + NW, ... (lane j
  // holding blocks j and j + 64, rs_n <= 128); requested here, with the first weight loads.
  constexpr int RB = 32 / NW;  // rows per wavefront (B <= 32)
  float rsv[RB][2];
  if (e.rs != nullptr) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int b = wids + r * NW;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = lane + 64 * h;
        rsv[r][h] = (b < B && j < e.rs_n) ? e.rs[b * e.rs_n + j] : 0.f;
      }
    }
  }
  // this wavefront's K steps s0 + wid, s0 + wid + NW, ... in batches of DEPTH
  for (int st0 = s0 + wids; st0 < s1; st0 += DEPTH * NW) {
    bf16x8 xb[DEPTH][4];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int st = st0 + d * NW;
      if (st < s1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (gv_lds_t)(&wl[wids][d][i * 512]), 16, voff[i],
                                                   st * GV_KB * 2, 0, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) xb[d][m] = b_ok ? *(const bf16x8*)(ap + st * GV_KB + 8 * m) : zero;
      }
    }
    __builtin_amdgcn_s_waitcnt(GV_VMCNT0);  // this wavefront's tiles are in LDS
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (st0 + d * NW < s1) {
        const bf16* base = &wl[wid][d][row * GV_KB];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 wa = *(const bf16x8*)(base + (((4 * g + m) ^ sw) << 3));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xb[d][m], acc, 0, 0, 0);
        }
      }
    }
  }
  // each wavefront's tile through its own LDS slots (read only by itself until here)
  float* const red = (float*)&wl[0][0][0];
  constexpr int RS = DEPTH * GV_ROWS * GV_KB / 2;  // floats per wavefront's slots (>= 64 * 16)
#pragma unroll
  for (int r = 0; r < 16; ++r) red[wid * RS + lane * 16 + r] = acc[r];
  if (e.rs != nullptr) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int b = wids + r * NW;
      if (b < B) {
        const float ss = wave_sum(rsv[r][0] + rsv[r][1]);
        if (lane == 0) rsc[b] = rsqrtf(ss / (float)K + e.eps);
      }
    }
  }
  __syncthreads();
  float v[64 * 16 / (NW * 64)];
#pragma unroll
  for (int i = 0; i < 64 * 16 / (NW * 64); ++i) {
    const int idx = threadIdx.x + i * NW * 64;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w * RS + idx];
    v[i] = t;
  }
  auto coords = [&](int idx, int& b, int& n) {
    const int l = idx >> 4, r = idx & 15;
    n = n0 + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
    b = l & 31;
  };
  if (e.rs != nullptr) {
#pragma unroll
    for (int i = 0; i < 64 * 16 / (NW * 64); ++i) {
      int b, n;
      coords(threadIdx.x + i * NW * 64, b, n);
      if (b < B) v[i] *= rsc[b];
    }
  }
  if (KS > 1) {
#pragma unroll
    for (int i = 0; i < 64 * 16 / (NW * 64); ++i) {
      int b, n;
      coords(threadIdx.x + i * NW * 64, b, n);
      if (b < B && n < N) partial[((size_t)ks * B + b) * N + n] = v[i];
    }
    return;
  }
  if (e.kind == DEC_RESID_RS) {
#pragma unroll
    for (int i = 0; i < 64 * 16 / (NW * 64); ++i) {
      int b, n;
      coords(threadIdx.x + i * NW * 64, b, n);
      float w = 0.f;
      if (b < B && n < N) {
        const size_t o = (size_t)b * e.ldo + n;
        w = ((float*)e.out)[o] + v[i];
        ((float*)e.out)[o] = w;
        e.xb[o] = (bf16)w;
      }
      sq[b][n - n0] = w * w;
    }
    __syncthreads();
    if ((int)threadIdx.x < B) {
      float ss = 0.f;
      for (int j = 0; j < GV_ROWS; ++j) ss += sq[threadIdx.x][j];
      e.ss[threadIdx.x * gridDim.x + blockIdx.x] = ss;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 64 * 16 / (NW * 64); ++i) {
    int b, n;
    coords(threadIdx.x + i * NW * 64, b, n);
    if (b < B && n < N) gv_apply<bf16>(e, b, n, v[i]);
  }
}

// fp32 weights and activations: one wavefront per output column n, lanes over K, all B rows.
__global__ __launch_bounds__(256) void gemv_f32_kernel(const float* __restrict__ act, int lda, int B,
                                                       const float* __restrict__ W0,
                                                       const float* __restrict__ W1,
                                                       const float* __restrict__ W2, int nseg0,
                                                       int nseg1, int N, int K, GvEpi e) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const float* w;
  if (n < nseg0) w = W0 + (size_t)n * K;
  else if (n < nseg0 + nseg1) w = W1 + (size_t)(n - nseg0) * K;
  else w = W2 + (size_t)(n - nseg0 - nseg1) * K;
  for (int b = 0; b < B; ++b) {
    const float* a = act + (size_t)b * lda;
    float s = 0.f;
    for (int k = lane; k < K; k += 64) s = fmaf(a[k], w[k], s);
    s = wave_sum(s);
    if (lane == 0) gv_apply<float>(e, b, n, s);
  }
}

// q/k/v of the step's token: RoPE at position pos[b] and per-head RMSNorm on the q and k heads
// (fp32, then one rounding to the cache type), q_hat to qout [B, H*D], k_hat and v into the
// cache at position pos[b].  One wavefront per (row, head) of the H + 2*Hkv heads; lane p
// rotates the pair (p, p + D/2).  The angle is formed as the forward's RoPE table forms it
// (fp64 power, cosine and sine, rounded to fp32).
constexpr int RA_KB = 16;  // partial tiles loaded together
template <typename AT>
__global__ __launch_bounds__(256) void rope_append_kernel(
    const float* __restrict__ y, int ldy, int KS, size_t kstride, const int32_t* __restrict__ pos,
    int B, int T, int H, int Hkv, int D, float eps, double base, AT* __restrict__ qout,
    AT* __restrict__ kc, AT* __restrict__ vc, unsigned* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int nh = H + 2 * Hkv;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= B * nh) return;
  const int b = w / nh, hh = w % nh, half = D >> 1;
  const int t = pos[b];
  if (t < 0 || t >= T) {
    if (lane == 0 && hh == 0) atomicOr(flags, GPT_FLAG_BAD_POS);
    return;
  }
  const float* src = y + (size_t)b * ldy + (size_t)hh * D;
  // The product's values at d0 and d1 (< D; d1 = -1: none): their K-split partial tiles summed
  // in split order, all tiles loaded before the first add so that the loads overlap.
  auto val2 = [&](int d0, int d1, float& v0, float& v1) {
    v0 = 0.f;
    v1 = 0.f;
    for (int k0 = 0; k0 < KS; k0 += RA_KB) {
      float t0[RA_KB], t1[RA_KB];
#pragma unroll
      for (int k = 0; k < RA_KB; ++k)
        if (k0 + k < KS) {
          t0[k] = src[(size_t)(k0 + k) * kstride + d0];
          t1[k] = d1 >= 0 ? src[(size_t)(k0 + k) * kstride + d1] : 0.f;
        }
#pragma unroll
      for (int k = 0; k < RA_KB; ++k)
        if (k0 + k < KS) {
          v0 = (k0 + k == 0) ? t0[k] : v0 + t0[k];
          v1 = (k0 + k == 0) ? t1[k] : v1 + t1[k];
        }
    }
  };
  if (hh >= H + Hkv) {  // v: copied into the cache
    const int g = hh - H - Hkv;
    AT* dst = vc + (((size_t)b * Hkv + g) * T + t) * D;
    for (int d = lane; d < D; d += 128) {
      float v0, v1;
      val2(d, d + 64 < D ? d + 64 : -1, v0, v1);
      dst[d] = from_f32<AT>(v0);
      if (d + 64 < D) dst[d + 64] = from_f32<AT>(v1);
    }
    return;
  }
  float y1 = 0.f, y2 = 0.f;
  if (lane < half) {
    const double omega = pow(base, -2.0 * (double)lane / (double)D);
    const double phi = (double)t * omega;
    const float c = (float)cos(phi), s = (float)sin(phi);
    float u1, u2;
    val2(lane, lane + half, u1, u2);
    y1 = u1 * c + u2 * s;
    y2 = -u1 * s + u2 * c;
  }
  const float ss = wave_sum(y1 * y1 + y2 * y2);
  const float r = rsqrtf(ss / (float)D + eps);
  AT* dst = hh < H ? qout + (size_t)b * H * D + (size_t)hh * D
                   : kc + (((size_t)b * Hkv + (hh - H)) * T + t) * D;
  if (lane < half) {
    dst[lane] = from_f32<AT>(y1 * r);
    dst[lane + half] = from_f32<AT>(y2 * r);
  }
}

// Attention of the step's queries over cached keys j in [lo, t], lo = max(0, t - w + 1), split
// over chunks of DA_CHUNK keys (flash-decoding): block (row b, KV head g, chunk c) scores the
// chunk's keys against the G = H/Hkv query heads that read KV head g (each key and value row is
// read once for the whole group), and writes per head the chunk's max m_c, sum l_c = sum_j
// exp(s_j - m_c) and unnormalised output O_c = sum_j exp(s_j - m_c) v_j (fp32).  The combine
// kernel merges the chunks: o = sum_c e^(m_c - m) O_c / sum_c e^(m_c - m) l_c.  Query head h
// reads KV head h*Hkv/H, i.e. the group of head h is h / G.
constexpr int DA_THREADS = 512;   // per chunk block (d24 decode step: 256 1.374 ms, 512 1.365, 1024 1.533)
constexpr int DA_CHUNK = 128;       // keys per block (d24 decode step with 512-thread blocks: 64 1.451 ms, 128 1.352, 256 1.373)
constexpr int DA_MAX_GROUP = 8;     // query heads per KV head


// Eight consecutive elements as loaded (bf16 or fp32), converted only where used, so that all of
// a thread's loads can be issued before the first of them is needed.
template <typename AT> struct Raw8;
template <> struct Raw8<bf16> { bf16x8 v; };
template <> struct Raw8<float> { f32x4 a, b; };
__device__ __forceinline__ void ld_raw(const bf16* p, Raw8<bf16>& r) { r.v = *(const bf16x8*)p; }
__device__ __forceinline__ void ld_raw(const float* p, Raw8<float>& r) {
  r.a = *(const f32x4*)p;
  r.b = *(const f32x4*)(p + 4);
}
__device__ __forceinline__ float raw_at(const Raw8<bf16>& r, int i) { return (float)r.v[i]; }
__device__ __forceinline__ float raw_at(const Raw8<float>& r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }

template <typename AT, int D>
__global__ __launch_bounds__(DA_THREADS) void decode_attn_chunk_kernel(
    const AT* __restrict__ q, const AT* __restrict__ kc, const AT* __restrict__ vc,
    const int32_t* __restrict__ pos, int T, int H, int Hkv, int window, float scale, int nch,
    float* __restrict__ part) {
  __shared__ float qs[DA_MAX_GROUP][D];
  __shared__ float sc[DA_MAX_GROUP][DA_CHUNK];
  __shared__ float ml[DA_MAX_GROUP][2];
  __shared__ float red[DA_THREADS / 64][DA_MAX_GROUP][D];
  const int c = blockIdx.y, bg = blockIdx.x, b = bg / Hkv, g = bg % Hkv;
  const int G = H / Hkv, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int t = pos[b];
  const bool ok = t >= 0 && t < T;
  const int lo = ok ? (t - window + 1 > 0 ? t - window + 1 : 0) : 0;
  const int j0 = lo + c * DA_CHUNK;
  const int nk = ok ? min(DA_CHUNK, t + 1 - j0) : 0;  // keys of this chunk (<= 0: none)
  // part layout per (b, h, chunk): [m, l, O[0..D)]
  auto slot = [&](int gi) { return part + (((size_t)b * H + g * G + gi) * nch + c) * (D + 2); };
  if (nk <= 0) {
    for (int i = tid; i < G * (D + 2); i += DA_THREADS) {
      const int gi = i / (D + 2), e = i % (D + 2);
      slot(gi)[e] = e == 0 ? -INFINITY : 0.f;
    }
    return;
  }
  // This thread's key chunks (score pass) and value rows (output pass) are requested first,
  // together, then the queries: one memory round trip instead of three.  Keys past the chunk's
  // end read the chunk's first key instead (their probability is 0).  Both passes load 16-byte
  // chunks (8 elements) with consecutive threads on consecutive chunks of a row, so that each
  // load instruction covers whole rows.
  constexpr int OCT = D / 8, PARTS = DA_THREADS / OCT;  // chunks per row; rows per instruction
  constexpr int VR = DA_CHUNK / PARTS;                  // key / value rows per thread
  const int oc = tid % OCT, pt = tid / OCT;
  Raw8<AT> kraw[VR], vraw[VR];
  {
    const AT* kb = kc + (((size_t)b * Hkv + g) * T + j0) * D + oc * 8;
    const AT* vb = vc + (((size_t)b * Hkv + g) * T + j0) * D + oc * 8;
#pragma unroll
    for (int k = 0; k < VR; ++k) {
      const int jv = pt + k * PARTS;
      ld_raw(kb + (size_t)(jv < nk ? jv : 0) * D, kraw[k]);
    }
#pragma unroll
    for (int k = 0; k < VR; ++k) {
      const int jv = pt + k * PARTS;
      ld_raw(vb + (size_t)(jv < nk ? jv : 0) * D, vraw[k]);
    }
  }
  for (int i = tid; i < G * D; i += DA_THREADS)
    qs[i / D][i % D] = to_f32(q[(size_t)b * H * D + (size_t)(g * G + i / D) * D + i % D]);
  __syncthreads();
  // scores: thread (chunk oc, rows pt + k * PARTS) forms 8-element partial dot products, summed
  // over the OCT threads of a row by DPP butterflies within 16-lane rows
  for (int gi = 0; gi < G; ++gi) {
    float qv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qs[gi][oc * 8 + i];
#pragma unroll
    for (int k = 0; k < VR; ++k) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s = fmaf(qv[i], raw_at(kraw[k], i), s);
      s += dpp<0xB1>(s);   // quad_perm [1,0,3,2]
      s += dpp<0x4E>(s);   // quad_perm [2,3,0,1]
      s += dpp<0x141>(s);  // row_half_mirror: 8-lane sums
      if constexpr (OCT == 16) s += dpp<0x140>(s);  // row_mirror: 16-lane sums
      const int jv = pt + k * PARTS;
      if (oc == 0) sc[gi][jv] = jv < nk ? s * scale : -INFINITY;
    }
  }
  __syncthreads();
  // per head: chunk max and sum (one wavefront per head, DA_CHUNK / 64 keys per lane)
  constexpr int KPL = DA_CHUNK / 64;
  for (int gi = wid; gi < G; gi += DA_THREADS / 64) {
    float a[KPL];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      a[k] = sc[gi][lane + 64 * k];
      mx = fmaxf(mx, a[k]);
    }
    const float m = wave_max(mx);
    float ps = 0.f;
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const float p = expf(a[k] - m);
      sc[gi][lane + 64 * k] = p;
      ps += p;
    }
    const float l = wave_sum(ps);
    if (lane == 0) { ml[gi][0] = m; ml[gi][1] = l; }
  }
  __syncthreads();
  // O = sum_j p_j v_j: thread (8-dimension octet, key part) reads 8 values of a row at once;
  // the value rows are read once for all heads of the group.  Parts are summed by shuffles
  // within a wavefront, then the block's wavefronts through LDS, in a fixed order.
  {
    float acc[DA_MAX_GROUP][8];
#pragma unroll
    for (int gi = 0; gi < DA_MAX_GROUP; ++gi)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[gi][i] = 0.f;
#pragma unroll
    for (int k = 0; k < VR; ++k) {
      const int jv = pt + k * PARTS;
      if (jv < nk) {
#pragma unroll
        for (int gi = 0; gi < DA_MAX_GROUP; ++gi)
          if (gi < G) {
            const float pj = sc[gi][jv];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[gi][i] = fmaf(pj, raw_at(vraw[k], i), acc[gi][i]);
          }
      }
    }
#pragma unroll
    for (int gi = 0; gi < DA_MAX_GROUP; ++gi)
      if (gi < G)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float a = acc[gi][i];
#pragma unroll
        for (int o = OCT; o < 64; o <<= 1) a += __shfl_xor(a, o);
        acc[gi][i] = a;
      }
    if (lane < OCT)
#pragma unroll
      for (int gi = 0; gi < DA_MAX_GROUP; ++gi)
        if (gi < G)
#pragma unroll
          for (int i = 0; i < 8; ++i) red[wid][gi][oc * 8 + i] = acc[gi][i];
    __syncthreads();
  }
  for (int i = tid; i < G * (D + 2); i += DA_THREADS) {
    const int gi = i / (D + 2), e = i % (D + 2);
    float v;
    if (e == 0) v = ml[gi][0];
    else if (e == 1) v = ml[gi][1];
    else {
      v = red[0][gi][e - 2];
#pragma unroll
      for (int w = 1; w < DA_THREADS / 64; ++w) v += red[w][gi][e - 2];
    }
    slot(gi)[e] = v;
  }
}

// o[b][h] = merge of the chunks' partial softmax results (fixed chunk order); rows with an
// invalid position get zeros (their logits are NaN).  The chunks' (m, l) are staged in LDS
// first so the output loop's loads are independent.
constexpr int DA_MAX_CHUNKS = 8192 / DA_CHUNK;

template <typename AT, int D>
__global__ __launch_bounds__(D) void decode_attn_combine_kernel(const float* __restrict__ part,
                                                                int nch, int H, AT* __restrict__ o) {
  __shared__ float wgt[DA_MAX_CHUNKS], lsum[DA_MAX_CHUNKS];
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* p = part + (size_t)bh * nch * (D + 2);
  for (int c = d; c < nch; c += D) { wgt[c] = p[c * (D + 2)]; lsum[c] = p[c * (D + 2) + 1]; }
  __syncthreads();
  float m = -INFINITY;
  for (int c = 0; c < nch; ++c) m = fmaxf(m, wgt[c]);
  float l = 0.f, acc = 0.f;
  if (m != -INFINITY)
    for (int c = 0; c < nch; ++c) {
      const float e = expf(wgt[c] - m);
      l = fmaf(e, lsum[c], l);
      acc = fmaf(e, p[c * (D + 2) + 2 + d], acc);
    }
  o[(size_t)bh * D + d] = from_f32<AT>(l > 0.f ? acc / l : 0.f);
}

// ----------------------------------------------------------------------------------- prefill
// The decode cache from one forward pass over P positions: k_hat rows (and, on the fp32 path,
// v rows) are copied from the forward's row-major [B*P][ld] projection at column col0 + g*D
// into [B][Hkv][T][D]; 16 bytes per thread.
template <typename AT>
__global__ __launch_bounds__(256) void cache_fill_rows_kernel(const AT* __restrict__ src, int ld,
                                                              int col0, AT* __restrict__ dst, int B,
                                                              int P, int T, int Hkv, int D) {
  constexpr int E = 16 / sizeof(AT);
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = Hkv * D / E;
  if (idx >= (long)B * P * per_row) return;
  const int c = (int)(idx % per_row), bt = (int)(idx / per_row), b = bt / P, t = bt % P;
  const int g = c / (D / E), d = (c % (D / E)) * E;
  *(u32x4*)(dst + (((size_t)b * Hkv + g) * T + t) * D + d) =
      *(const u32x4*)(src + (size_t)bt * ld + col0 + g * D + d);
}

// bf16 path: v of the forward is stored transposed, [B][Hkv][D][P]; 64x64 tiles go through LDS
// to [B][Hkv][T][D].
__global__ __launch_bounds__(256) void cache_fill_vt_kernel(const bf16* __restrict__ vt,
                                                            bf16* __restrict__ dst, int P, int T,
                                                            int D) {
  __shared__ bf16 tile[64][64 + 2];
  const int bg = blockIdx.z, d0 = blockIdx.y * 64, t0 = blockIdx.x * 64;
  const bf16* s = vt + (size_t)bg * D * P;
  bf16* o = dst + (size_t)bg * T * D;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int dd = i / 64, tt = i % 64;
    if (d0 + dd < D && t0 + tt < P) tile[dd][tt] = s[(size_t)(d0 + dd) * P + t0 + tt];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int tt = i / 64, dd = i % 64;
    if (d0 + dd < D && t0 + tt < P) o[(size_t)(t0 + tt) * D + d0 + dd] = tile[dd][tt];
  }
}

// Row b's last prompt position r = b*P + len_b - 1 (len_b = lens[b], or P), RMS-normalised in
// fp32 from the residual stream x and rounded once to the activation type; an invalid length
// raises GPT_FLAG_BAD_POS and gives a NaN row (so its logits are NaN).
template <typename AT>
__global__ __launch_bounds__(64) void last_row_norm_kernel(const float* __restrict__ x,
                                                           const int32_t* __restrict__ lens, int P,
                                                           int C, float eps, AT* __restrict__ out,
                                                           unsigned* __restrict__ flags) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int len = lens != nullptr ? lens[b] : P;
  AT* o = out + (size_t)b * C;
  if (len < 1 || len > P) {
    if (lane == 0) atomicOr(flags, GPT_FLAG_BAD_POS);
    for (int i = lane; i < C; i += 64) o[i] = from_f32<AT>(__builtin_nanf(""));
    return;
  }
  const float* xr = x + ((size_t)b * P + len - 1) * C;
  float ss = 0.f;
  for (int i = lane; i < C; i += 64) ss += xr[i] * xr[i];
  const float r = rsqrtf(wave_sum(ss) / (float)C + eps);
  for (int i = lane; i < C; i += 64) o[i] = from_f32<AT>(xr[i] * r);
}

// ---------------------------------------------------------------------------------- sampling
constexpr int SMP_THREADS = 1024;

__device__ __forceinline__ unsigned order_key(float f) {  // monotone map float -> uint32
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One block per row.  Temperature 0: the first index of the largest logit.  Otherwise the
// k-th largest logit (exact radix select over the order-preserving 32-bit keys, 8 bits per
// pass) bounds the kept set {v : z_v >= z_(k)}; p_v = exp((z_v - max) / tau) over it; the token
// is the first v, in vocabulary order, whose running sum exceeds u * sum_v p_v.  Each thread
// owns a contiguous run of the vocabulary; runs are summed by a block scan, so the total and
// the running sums come from the same additions.
__global__ __launch_bounds__(SMP_THREADS) void sample_kernel(const float* __restrict__ logits,
                                                             int V, int top_k, float temperature,
                                                             const float* __restrict__ u,
                                                             int32_t* __restrict__ out) {
  __shared__ unsigned hist[256];
  __shared__ float scratch[SMP_THREADS / 64];
  __shared__ float runs[SMP_THREADS];
  __shared__ unsigned sel[2];
  __shared__ unsigned long long best, last_kept;
  const int b = blockIdx.x, tid = threadIdx.x;
  const float* z = logits + (size_t)b * V;
  const int per = (V + SMP_THREADS - 1) / SMP_THREADS;
  const int v0 = tid * per, v1 = min(V, v0 + per);
  if (temperature == 0.f) {  // argmax, first index on ties: max of (key, ~index)
    unsigned long long m = 0;
    for (int v = v0; v < v1; ++v) {
      const unsigned long long c = ((unsigned long long)order_key(z[v]) << 32) | (unsigned)(~v);
      m = c > m ? c : m;
    }
    if (tid == 0) best = 0;
    __syncthreads();
    atomicMax(&best, m);
    __syncthreads();
    if (tid == 0) out[b] = (int32_t)(~(unsigned)(best & 0xffffffffu));
    return;
  }
  // threshold key of the k-th largest logit (0 = keep all)
  unsigned thr = 0;
  if (top_k > 0 && top_k < V) {
    unsigned prefix = 0, mask = 0;
    int need = top_k;  // rank still to find among keys matching the prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += SMP_THREADS) hist[i] = 0;
      __syncthreads();
      for (int v = v0; v < v1; ++v) {
        const unsigned k = order_key(z[v]);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1u);
      }
      __syncthreads();
      if (tid == 0) {  // digit holding the need-th largest, scanning from the top
        int acc = 0, dgt = 255;
        for (; dgt > 0; --dgt) {
          if (acc + (int)hist[dgt] >= need) break;
          acc += hist[dgt];
        }
        sel[0] = (unsigned)dgt;
        sel[1] = (unsigned)(need - acc);
      }
      __syncthreads();
      prefix |= sel[0] << shift;
      mask |= 255u << shift;
      need = (int)sel[1];
      __syncthreads();
    }
    thr = prefix;  // every bit decided: the exact key of the k-th largest
  }
  float mloc = -INFINITY;
  for (int v = v0; v < v1; ++v) mloc = fmaxf(mloc, z[v]);
  mloc = wave_max(mloc);
  __syncthreads();
  if ((tid & 63) == 0) scratch[tid >> 6] = mloc;
  __syncthreads();
  float mx = scratch[0];
  for (int w = 1; w < SMP_THREADS / 64; ++w) mx = fmaxf(mx, scratch[w]);
  const float inv_t = 1.f / temperature;
  float run = 0.f;
  for (int v = v0; v < v1; ++v)
    if (order_key(z[v]) >= thr) run += expf((z[v] - mx) * inv_t);
  __syncthreads();
  runs[tid] = run;
  __syncthreads();
  // exclusive scan of the runs (thread 0, fixed order; 1024 additions)
  if (tid == 0) {
    float acc = 0.f;
    for (int i = 0; i < SMP_THREADS; ++i) { const float r = runs[i]; runs[i] = acc; acc += r; }
    scratch[0] = acc;
    best = ~0ull;
    last_kept = 0ull;
  }
  __syncthreads();
  const float total = scratch[0], target = u[b] * total;
  float s = runs[tid];
  int pick = -1, last = -1;
  for (int v = v0; v < v1; ++v) {
    if (order_key(z[v]) < thr) continue;
    last = v;
    s += expf((z[v] - mx) * inv_t);
    if (s > target) { pick = v; break; }
  }
  if (pick >= 0) atomicMin(&best, (unsigned long long)pick);
  if (last >= 0) atomicMax(&last_kept, (unsigned long long)last + 1);
  __syncthreads();
  // no running sum exceeded u * total (u * total rounded up to the total): the last kept token
  if (tid == 0) out[b] = best != ~0ull ? (int32_t)best : (int32_t)last_kept - 1;
}

}  // namespace

// K splits of a product: enough blocks to keep every CU busy, each split with >= 8 K steps (one
// per wavefront of an 8-wavefront block).  At d24 (q/k/v 3 splits, MLP down 12), against 4-
// wavefront blocks and twice the splits: decode step 1.368 -> 1.353 ms, alternated on one box;
// the same halved splits on 4 wavefronts with two steps each were 0.7 % slower.
int gemv_splits(int N, int K) {
  const int nrb = (N + GV_ROWS - 1) / GV_ROWS, nks = K / GV_KB;
  int ks = (GV_TARGET_BLOCKS + nrb - 1) / nrb;
  ks = ks < nks / (2 * GV_WAVES) ? ks : nks / (2 * GV_WAVES);
  return ks > 1 ? ks : 1;
}

hipError_t launch_gemv(bool bf, int kind, const void* act, int lda, int B, const void* W0,
                       const void* W1, const void* W2, int nseg0, int nseg1, int N, int K,
                       void* out, int ldo, hipStream_t s, int KS, float* partial, float cap,
                       const int32_t* pos, const int32_t* tokens, int T, int V, const float* rs,
                       int rs_n, float eps, void* xb, float* ss) {
  if (B < 1 || B > 32 || N < 1 || K < 1 || K % GV_KB || KS < 1) return hipErrorInvalidValue;
  if ((rs != nullptr || kind == DEC_RESID_RS) && !bf) return hipErrorInvalidValue;
  if (rs != nullptr && (rs_n < 1 || rs_n > 128)) return hipErrorInvalidValue;
  if (kind == DEC_RESID_RS && (KS != 1 || xb == nullptr || ss == nullptr)) return hipErrorInvalidValue;
  if ((nseg0 < N && nseg0 % GV_ROWS) || (nseg0 + nseg1 < N && (nseg0 + nseg1) % GV_ROWS))
    return hipErrorInvalidValue;  // interior segment boundaries on block boundaries
  GvEpi e{kind, out, ldo, cap, pos, tokens, T, V, rs, rs_n, eps, (bf16*)xb, ss};
  if (bf) {
    if (KS > 1 && !partial) return hipErrorInvalidValue;
    const int grid = (N + GV_ROWS - 1) / GV_ROWS * KS;
    // K steps of the largest split: up to 4 on 4 wavefronts, up to 8 on 8 (one step each, 32 KB
    // of LDS); longer ranges (the unsplit out-projection, MLP-up and lm_head products) on 8
    // wavefronts with two steps each in flight per batch (64 KB: two blocks per CU).  Measured
    // at the d24 shapes with the weights cold (MLP up / lm_head): 4 x 6 steps 6.9 / 25.3 us,
    // 8 x 3 6.4 / 23.5 us, 8 x 2 6.4 / 19.2 us, 16 x 2 6.3 / 22.7 us.
    const int steps = (K / GV_KB + KS - 1) / KS;
#define GPTK_GV(NW, DEPTH)                                                                          \
  gemv_bf16_kernel<NW, DEPTH><<<grid, NW * 64, 0, s>>>(                                             \
      (const bf16*)act, lda, B, (const bf16*)W0, (const bf16*)W1, (const bf16*)W2, nseg0, nseg1, N, \
      K, KS, partial, e)
    if (steps <= GV_WAVES) GPTK_GV(GV_WAVES, 1);
    else if (steps <= 8) GPTK_GV(8, 1);
    else GPTK_GV(8, 2);
#undef GPTK_GV
  } else {
    if (KS != 1) return hipErrorInvalidValue;
    gemv_f32_kernel<<<(N + 3) / 4, 256, 0, s>>>((const float*)act, lda, B, (const float*)W0,
                                                (const float*)W1, (const float*)W2, nseg0, nseg1,
                                                N, K, e);
  }
  return hipGetLastError();
}


hipError_t launch_rope_append(bool bf, const float* y, int ldy, int KS, const int32_t* pos, int B,
                              int T, int H, int Hkv, int D, float eps, float base, void* qout,
                              void* kc, void* vc, unsigned* flags, hipStream_t s) {
  const int grid = (B * (H + 2 * Hkv) + 3) / 4;
  const size_t kstride = (size_t)B * ldy;
  if (bf)
    rope_append_kernel<bf16><<<grid, 256, 0, s>>>(y, ldy, KS, kstride, pos, B, T, H, Hkv, D, eps,
                                                  (double)base, (bf16*)qout, (bf16*)kc, (bf16*)vc,
                                                  flags);
  else
    rope_append_kernel<float><<<grid, 256, 0, s>>>(y, ldy, KS, kstride, pos, B, T, H, Hkv, D, eps,
                                                   (double)base, (float*)qout, (float*)kc,
                                                   (float*)vc, flags);
  return hipGetLastError();
}

int decode_attn_chunks(int T) { return (T + DA_CHUNK - 1) / DA_CHUNK; }

hipError_t launch_decode_attn(bool bf, const void* q, const void* kc, const void* vc,
                              const int32_t* pos, int B, int T, int H, int Hkv, int D, int window,
                              float scale, void* o, float* part, hipStream_t s) {
  if ((D != 64 && D != 128) || H % Hkv || H / Hkv > DA_MAX_GROUP || decode_attn_chunks(T) > DA_MAX_CHUNKS)
    return hipErrorInvalidValue;
  const int w = window < T ? window : T;
  const int nch = (w + DA_CHUNK - 1) / DA_CHUNK;  // chunks a window spans (partials laid out per nch)
  const dim3 grid(B * Hkv, nch);
#define GPTK_DA(AT, DD)                                                                              \
  do {                                                                                               \
    decode_attn_chunk_kernel<AT, DD><<<grid, DA_THREADS, 0, s>>>((const AT*)q, (const AT*)kc,         \
                                                                 (const AT*)vc, pos, T, H, Hkv, w,    \
                                                                 scale, nch, part);                  \
    decode_attn_combine_kernel<AT, DD><<<B * H, DD, 0, s>>>(part, nch, H, (AT*)o);                   \
  } while (0)
  if (bf) { if (D == 128) GPTK_DA(bf16, 128); else GPTK_DA(bf16, 64); }
  else { if (D == 128) GPTK_DA(float, 128); else GPTK_DA(float, 64); }
#undef GPTK_DA
  return hipGetLastError();
}

hipError_t launch_cache_fill(bool bf, const void* qk, int ld, int kcol0, const void* vsrc,
                             int vcol0, int B, int P, int T, int Hkv, int D, void* kc, void* vc,
                             hipStream_t s) {
  const long n = (long)B * P * Hkv * D / (bf ? 8 : 4);
  const int grid = (int)((n + 255) / 256);
  if (bf) {
    cache_fill_rows_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)qk, ld, kcol0, (bf16*)kc, B, P, T, Hkv, D);
    const dim3 g2((P + 63) / 64, (D + 63) / 64, B * Hkv);
    cache_fill_vt_kernel<<<g2, 256, 0, s>>>((const bf16*)vsrc, (bf16*)vc, P, T, D);
  } else {
    cache_fill_rows_kernel<float><<<grid, 256, 0, s>>>((const float*)qk, ld, kcol0, (float*)kc, B, P, T, Hkv, D);
    cache_fill_rows_kernel<float><<<grid, 256, 0, s>>>((const float*)vsrc, ld, vcol0, (float*)vc, B, P, T, Hkv, D);
  }
  return hipGetLastError();
}

hipError_t launch_last_row_norm(bool bf, const float* x, const int32_t* lens, int B, int P, int C,
                                float eps, void* out, unsigned* flags, hipStream_t s) {
  if (bf) last_row_norm_kernel<bf16><<<B, 64, 0, s>>>(x, lens, P, C, eps, (bf16*)out, flags);
  else last_row_norm_kernel<float><<<B, 64, 0, s>>>(x, lens, P, C, eps, (float*)out, flags);
  return hipGetLastError();
}

hipError_t launch_sample(const float* logits, int B, int V, int top_k, float temperature,
                         const float* u, int32_t* out, hipStream_t s) {
  if (B < 1 || V < 1) return hipErrorInvalidValue;
  sample_kernel<<<B, SMP_THREADS, 0, s>>>(logits, V, top_k, temperature, u, out);
  return hipGetLastError();
}

}  // namespace gptk
