// Row-wise HBM-bound kernels: embedding gather + RMSNorm, residual x0-mix + RMSNorm, the RoPE
// table, and RoPE + per-head RMSNorm (QK-norm).  One 64-lane wavefront owns one row and reduces
// its sum of squares with cross-lane shuffles; statistics are fp32.
//
// Sources: "The Mathematics of Karpathy's nanochat", sections "High-Level Forward Pass" (embed,
// norm, keep x0), "RMS Normalization", "Residual Stream with Learnable Scalars" (x <- lambda x +
// mu x0), "Rotary Position Embeddings (RoPE)" and "QK-Norm with Sharpening"; the two-block
// PrefixRMSNorm of the nested model: "Fully Nested Transformers", opening section.  The prefix
// statistic is the same lane-ordered partial sum over columns [0, c1) that a row of width c1
// accumulates, so the first block of a nested row normalises exactly as a standalone row of
// that width does.
#include "common.h"
#include "kernels.h"

namespace gptk {
namespace {

constexpr int ROWS_PER_BLOCK = 4;  // 4 wavefronts of 64 lanes

__device__ __forceinline__ void load4(const float* p, float v[4]) {
  float4 t = *(const float4*)p;
  v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4(const bf16* p, float v[4]) {
  bf16x4 t = *(const bf16x4*)p;
  v[0] = (float)t[0]; v[1] = (float)t[1]; v[2] = (float)t[2]; v[3] = (float)t[3];
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float v[4]) {
  bf16x4 t;
  t[0] = (bf16)v[0]; t[1] = (bf16)v[1]; t[2] = (bf16)v[2]; t[3] = (bf16)v[3];
  *(bf16x4*)p = t;
}

// NCH = number of 4-element chunks per lane (C <= 256 * NCH).
template <typename WT, typename AT, int NCH>
__global__ __launch_bounds__(256) void embed_norm_kernel(
    const int32_t* __restrict__ tokens, const WT* __restrict__ wte, const float* __restrict__ lam,
    const float* __restrict__ mu, float* __restrict__ x0, float* __restrict__ x, AT* __restrict__ xn,
    int M, int C, int V, float eps, unsigned* __restrict__ flags, const WT* __restrict__ pe, int c1) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (row >= M) return;
  int t = tokens[row];
  if ((unsigned)t >= (unsigned)V) {  // out-of-range id: flag it, read row 0 so nothing faults
    if (lane == 0) atomicOr(flags, GPT_FLAG_BAD_TOKEN);
    t = 0;
  }
  const WT* src = wte + (size_t)t * C;
  float v[NCH][4];
  float ss = 0.f, ss1 = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = (c * 64 + lane) * 4;
    if (i < C) {
      load4(src + i, v[c]);
      if (pe != nullptr) {  // per-pass embedding of the looped trunk, added before the norm
        float pv[4];
        load4(pe + i, pv);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[c][k] += pv[k];
      }
      const float q = v[c][0] * v[c][0] + v[c][1] * v[c][1] + v[c][2] * v[c][2] + v[c][3] * v[c][3];
      ss += q;
      if (i < c1) ss1 += q;
    }
  }
  ss = wave_sum(ss);
  ss1 = c1 < C ? wave_sum(ss1) : ss;
  const float r0 = rsqrtf(ss / (float)C + eps), r01 = rsqrtf(ss1 / (float)c1 + eps);
  const float a = lam[0], b = mu[0];
  float ss2 = 0.f, ss21 = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = (c * 64 + lane) * 4;
    if (i < C) {
      float e0[4], e1[4];
      const float rr = i < c1 ? r01 : r0;
      float q = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        e0[k] = v[c][k] * rr;
        e1[k] = a * e0[k] + b * e0[k];
        q += e1[k] * e1[k];
        v[c][k] = e1[k];
      }
      ss2 += q;
      if (i < c1) ss21 += q;
      store4(x0 + (size_t)row * C + i, e0);
      store4(x + (size_t)row * C + i, e1);
    }
  }
  ss2 = wave_sum(ss2);
  ss21 = c1 < C ? wave_sum(ss21) : ss2;
  const float r1 = rsqrtf(ss2 / (float)C + eps), r11 = rsqrtf(ss21 / (float)c1 + eps);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = (c * 64 + lane) * 4;
    if (i < C) {
      float e[4];
      const float rr = i < c1 ? r11 : r1;
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = v[c][k] * rr;
      store4(xn + (size_t)row * C + i, e);
    }
  }
}

template <typename AT, int NCH, bool MIX>
__global__ __launch_bounds__(256) void mix_norm_kernel(
    float* __restrict__ x, const float* __restrict__ x0, const float* __restrict__ lam,
    const float* __restrict__ mu, int layer, AT* __restrict__ xn, int M, int C, float eps, int c1) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (row >= M) return;
  float* xr = x + (size_t)row * C;
  float a = 1.f, b = 0.f;
  if (MIX) { a = lam[layer]; b = mu[layer]; }
  float v[NCH][4];
  float ss = 0.f, ss1 = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = (c * 64 + lane) * 4;
    if (i < C) {
      load4(xr + i, v[c]);
      if (MIX) {
        float w[4];
        load4(x0 + (size_t)row * C + i, w);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[c][k] = a * v[c][k] + b * w[k];
        store4(xr + i, v[c]);
      }
      const float q = v[c][0] * v[c][0] + v[c][1] * v[c][1] + v[c][2] * v[c][2] + v[c][3] * v[c][3];
      ss += q;
      if (i < c1) ss1 += q;
    }
  }
  ss = wave_sum(ss);
  ss1 = c1 < C ? wave_sum(ss1) : ss;
  const float r = rsqrtf(ss / (float)C + eps), r1 = rsqrtf(ss1 / (float)c1 + eps);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int i = (c * 64 + lane) * 4;
    if (i < C) {
      float e[4];
      const float rr = i < c1 ? r1 : r;
#pragma unroll
      for (int k = 0; k < 4; ++k) e[k] = v[c][k] * rr;
      store4(xn + (size_t)row * C + i, e);
    }
  }
}

// Rows of x after a K-split product, each row spread over blocks of AMR_COLS columns (few rows,
// long partial sums): x += sum_k add[k] (the partials of a chunk all loaded, AMN_KB at a time,
// before any is added, then summed over four interleaved accumulators -- k into k mod 4,
// combined pairwise), then the optional x0 mix x = lam[layer] x + mu[layer] x0.  Writes x,
// xb = bf16(x) and the block's sum of squares of its columns of x, ss[row * nblk + blk] (per
// thread its 4 columns in order, then a wavefront butterfly); the consuming product applies the
// row scale 1/rms from those sums.
constexpr int AMN_KB = 32, AMR_COLS = 256;
__global__ __launch_bounds__(64) void add_mix_rows_kernel(float* __restrict__ x,
                                                          const float* __restrict__ add, int ks,
                                                          const float* __restrict__ x0,
                                                          const float* __restrict__ lam,
                                                          const float* __restrict__ mu, int layer,
                                                          bool mix, bf16* __restrict__ xb,
                                                          float* __restrict__ ss, int M, int C) {
  const int blk = blockIdx.x, row = blockIdx.y;
  const int i = blk * AMR_COLS + 4 * threadIdx.x;
  float q = 0.f;
  if (i < C) {
    float* const xr = x + (size_t)row * C + i;
    const f32x4 xv = *(const f32x4*)xr;
    const f32x4 x0v = mix ? *(const f32x4*)(x0 + (size_t)row * C + i) : f32x4{};
    f32x4 y4[4] = {};
    for (int k0 = 0; k0 < ks; k0 += AMN_KB) {
      f32x4 t[AMN_KB];
#pragma unroll
      for (int k = 0; k < AMN_KB; ++k)
        if (k0 + k < ks) t[k] = *(const f32x4*)(add + ((size_t)(k0 + k) * M + row) * C + i);
#pragma unroll
      for (int k = 0; k < AMN_KB; ++k)
        if (k0 + k < ks) y4[k & 3] += t[k];  // AMN_KB is a multiple of 4: (k0 + k) & 3 == k & 3
    }
    const f32x4 y = (y4[0] + y4[1]) + (y4[2] + y4[3]);
    f32x4 w = xv + y;
    if (mix) w = lam[layer] * w + mu[layer] * x0v;
    *(f32x4*)xr = w;
    bf16x4 wb;
#pragma unroll
    for (int k = 0; k < 4; ++k) wb[k] = (bf16)w[k];
    *(bf16x4*)(xb + (size_t)row * C + i) = wb;
    q = w[0] * w[0] + w[1] * w[1] + w[2] * w[2] + w[3] * w[3];
  }
  q = wave_sum(q);
  if (threadIdx.x == 0) ss[(size_t)row * gridDim.x + blk] = q;
}

__global__ void rope_table_kernel(float2* __restrict__ cs, int T, int half, double base) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * half) return;
  const int t = idx / half, j = idx % half;
  const double omega = pow(base, -2.0 * (double)j / (double)(2 * half));
  const double phi = (double)t * omega;
  cs[idx] = make_float2((float)cos(phi), (float)sin(phi));
}

// One wavefront per (row, head); lane p rotates the pair (p, p + D/2).
template <typename AT>
__global__ __launch_bounds__(256) void qk_rope_norm_kernel(AT* __restrict__ qk, int ld,
                                                           const float2* __restrict__ cs, int M,
                                                           int T, int nheads, int D, float eps) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  const int row = (int)(w / nheads), hh = (int)(w % nheads);
  if (row >= M) return;
  const int t = row % T, half = D >> 1;
  AT* p = qk + (size_t)row * ld + (size_t)hh * D;
  float y1 = 0.f, y2 = 0.f;
  if (lane < half) {
    const float u1 = to_f32(p[lane]), u2 = to_f32(p[lane + half]);
    const float2 c = cs[t * half + lane];
    y1 = u1 * c.x + u2 * c.y;
    y2 = -u1 * c.y + u2 * c.x;
  }
  const float ss = wave_sum(y1 * y1 + y2 * y2);
  const float r = rsqrtf(ss / (float)D + eps);
  if (lane < half) {
    p[lane] = from_f32<AT>(y1 * r);
    p[lane + half] = from_f32<AT>(y2 * r);
  }
}

template <typename F>
hipError_t dispatch_nch(int C, F&& f) {
  if (C <= 256) return f(std::integral_constant<int, 1>{});
  if (C <= 512) return f(std::integral_constant<int, 2>{});
  if (C <= 1024) return f(std::integral_constant<int, 4>{});
  if (C <= 2048) return f(std::integral_constant<int, 8>{});
  if (C <= 4096) return f(std::integral_constant<int, 16>{});
  if (C <= 8192) return f(std::integral_constant<int, 32>{});
  return hipErrorInvalidValue;
}

// Value embedding of the fp32 path ("The Mathematics of Karpathy's nanochat", section "Value
// Embeddings (ResFormer)"): one wavefront per token; each KV head's gate is 3 sigmoid of the
// first 12 normalised input channels against that head's gate row, then v += gate * ve[token].
__global__ __launch_bounds__(256) void ve_mix_f32_kernel(float* __restrict__ qkv, int ld, int voff,
                                                         const float* __restrict__ xn, int ldx,
                                                         const int32_t* __restrict__ tokens, int vocab,
                                                         const float* __restrict__ ve,
                                                         const float* __restrict__ gate, int M,
                                                         int Hkv, int D) {
  const int row = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;
  int tk = tokens[row];
  tk = (tk >= 0 && tk < vocab) ? tk : 0;
  const float* xr = xn + (size_t)row * ldx;
  float* vr = qkv + (size_t)row * ld + voff;
  const float* er = ve + (size_t)tk * Hkv * D;
  for (int h = 0; h < Hkv; ++h) {
    float z = 0.f;
    for (int c = 0; c < 12; ++c) z = fmaf(xr[c], gate[h * 12 + c], z);
    const float gv = 3.f / (1.f + expf(-z));
    for (int d = lane; d < D; d += 64) vr[h * D + d] += gv * er[h * D + d];
  }
}

}  // namespace

hipError_t launch_rope_table(float2* cs, int T, int D, float base, hipStream_t s) {
  const int n = T * (D / 2);
  rope_table_kernel<<<(n + 255) / 256, 256, 0, s>>>(cs, T, D / 2, (double)base);
  return hipGetLastError();
}

hipError_t launch_embed_norm(const int32_t* tokens, const void* wte, bool wbf16, const float* lam,
                             const float* mu, float* x0, float* x, void* xn, int M, int C, int V,
                             float eps, unsigned* flags, hipStream_t s, const void* pe, int c1) {
  if (c1 <= 0) c1 = C;
  if (C % 4 || c1 % 4 || c1 > C) return hipErrorInvalidValue;
  const int grid = (M + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  return dispatch_nch(C, [&](auto nch) {
    constexpr int N = decltype(nch)::value;
    if (wbf16)
      embed_norm_kernel<bf16, bf16, N><<<grid, 256, 0, s>>>(tokens, (const bf16*)wte, lam, mu, x0, x,
                                                            (bf16*)xn, M, C, V, eps, flags,
                                                            (const bf16*)pe, c1);
    else
      embed_norm_kernel<float, float, N><<<grid, 256, 0, s>>>(tokens, (const float*)wte, lam, mu, x0,
                                                              x, (float*)xn, M, C, V, eps, flags,
                                                              (const float*)pe, c1);
    return hipGetLastError();
  });
}

int add_mix_rows_blocks(int C) { return (C + AMR_COLS - 1) / AMR_COLS; }

hipError_t launch_add_mix_rows(float* x, const float* add, int ks, const float* x0, const float* lam,
                               const float* mu, int layer, bool mix, void* xb, float* ss, int M,
                               int C, hipStream_t s) {
  if (C % 4 || ks < 0 || (ks > 0 && add == nullptr) || M < 1) return hipErrorInvalidValue;
  add_mix_rows_kernel<<<dim3(add_mix_rows_blocks(C), M), 64, 0, s>>>(x, add, ks, x0, lam, mu, layer, mix,
                                                                    (bf16*)xb, ss, M, C);
  return hipGetLastError();
}

hipError_t launch_mix_norm(float* x, const float* x0, const float* lam, const float* mu, int layer,
                           bool mix, void* xn, bool xbf16, int M, int C, float eps, hipStream_t s,
                           int c1) {
  if (c1 <= 0) c1 = C;
  if (C % 4 || c1 % 4 || c1 > C) return hipErrorInvalidValue;
  const int grid = (M + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  return dispatch_nch(C, [&](auto nch) {
    constexpr int N = decltype(nch)::value;
    if (xbf16) {
      if (mix) mix_norm_kernel<bf16, N, true><<<grid, 256, 0, s>>>(x, x0, lam, mu, layer, (bf16*)xn, M, C, eps, c1);
      else mix_norm_kernel<bf16, N, false><<<grid, 256, 0, s>>>(x, x0, lam, mu, layer, (bf16*)xn, M, C, eps, c1);
    } else {
      if (mix) mix_norm_kernel<float, N, true><<<grid, 256, 0, s>>>(x, x0, lam, mu, layer, (float*)xn, M, C, eps, c1);
      else mix_norm_kernel<float, N, false><<<grid, 256, 0, s>>>(x, x0, lam, mu, layer, (float*)xn, M, C, eps, c1);
    }
    return hipGetLastError();
  });
}

hipError_t launch_ve_mix_f32(float* qkv, int ld, int voff, const float* xn, int ldx,
                             const int32_t* tokens, int vocab, const float* ve, const float* gate,
                             int M, int Hkv, int D, hipStream_t s) {
  const int grid = (M + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  ve_mix_f32_kernel<<<grid, 256, 0, s>>>(qkv, ld, voff, xn, ldx, tokens, vocab, ve, gate, M, Hkv, D);
  return hipGetLastError();
}

hipError_t launch_qk_rope_norm(void* qk, bool bf16_, int ld, const float2* cs, int M, int T,
                               int nheads, int D, float eps, hipStream_t s) {
  if (D > 128 || (D & 1)) return hipErrorInvalidValue;
  const long waves = (long)M * nheads;
  const int grid = (int)((waves + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK);
  if (bf16_)
    qk_rope_norm_kernel<bf16><<<grid, 256, 0, s>>>((bf16*)qk, ld, cs, M, T, nheads, D, eps);
  else
    qk_rope_norm_kernel<float><<<grid, 256, 0, s>>>((float*)qk, ld, cs, M, T, nheads, D, eps);
  return hipGetLastError();
}

}  // namespace gptk
