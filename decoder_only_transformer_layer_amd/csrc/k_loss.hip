// Per-token cross-entropy from the fused lm_head epilogue's partial sums, and the mean loss.
//
// Source: "The Mathematics of Karpathy's nanochat", section "Cross-Entropy Loss": the loss of a
// position is log(sum_v exp(zhat_v)) - zhat_target, positions whose target is -1 are excluded,
// and the batch loss is the mean over the kept positions.  With softcapped logits every
// zhat <= cap, so log(sum_v exp(zhat_v)) = cap + log(sum_v exp(zhat_v - cap)) needs no running
// maximum: each term lies in [exp(-2 cap), 1].
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace gptk {
namespace {

__global__ __launch_bounds__(256) void ce_finalize_kernel(
    const float* __restrict__ partial, int nnb, const float* __restrict__ tgt_logit,
    const int32_t* __restrict__ targets, const int32_t* __restrict__ tokens, int M, int V, float cap,
    float* __restrict__ loss, unsigned* __restrict__ flags) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  float s = 0.f;
  for (int i = lane; i < nnb; i += 64) s += partial[(size_t)row * nnb + i];
  s = wave_sum(s);
  if (lane != 0) return;
  const int y = targets[row];
  const int t = tokens[row];
  float l;
  if (y == -1) {
    l = 0.f;
  } else if ((unsigned)y >= (unsigned)V) {
    atomicOr(flags, GPT_FLAG_BAD_TARGET);
    l = NAN;
  } else {
    l = cap + logf(s) - cap * tanhf(tgt_logit[row] / cap);
  }
  if ((unsigned)t >= (unsigned)V) l = NAN;  // flagged by the embedding kernel
  loss[row] = l;
}

// One block; fixed summation order so repeated calls give identical bits.
__global__ __launch_bounds__(1024) void ce_mean_kernel(const float* __restrict__ loss,
                                                       const int32_t* __restrict__ targets, int M,
                                                       float* __restrict__ mean) {
  __shared__ double ssum[1024];
  __shared__ int scnt[1024];
  const int tid = threadIdx.x;
  double s = 0.0;
  int n = 0;
  for (int i = tid; i < M; i += 1024) {
    if (targets[i] != -1) { s += (double)loss[i]; ++n; }
  }
  ssum[tid] = s;
  scnt[tid] = n;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (tid < w) { ssum[tid] += ssum[tid + w]; scnt[tid] += scnt[tid + w]; }
    __syncthreads();
  }
  if (tid == 0) *mean = scnt[0] > 0 ? (float)(ssum[0] / (double)scnt[0]) : NAN;
}

// Raw logit of each row's target from the first c1 columns of the row and of the target's W_U
// row (bf16 operands, fp32 sum), one wavefront per row: the kfront=1 logit of a nested model,
// whose cross-entropy sums the lm_head pass takes at K = c1 ("Fully Nested Transformers": the
// prefix cross-entropy).  Rows whose target is -1 or out of range get 0 (the loss kernel reports
// them).
__global__ __launch_bounds__(256) void prefix_target_logit_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ wu, const int32_t* __restrict__ targets,
    int M, int C, int c1, int V, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const int y = targets[row];
  float s = 0.f;
  if (y >= 0 && y < V) {
    const bf16* xr = x + (size_t)row * C;
    const bf16* wr = wu + (size_t)y * C;
    for (int k = lane * 8; k < c1; k += 64 * 8) {
      const bf16x8 a = *(const bf16x8*)(xr + k), b = *(const bf16x8*)(wr + k);
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf((float)a[e], (float)b[e], s);
    }
  }
  s = wave_sum(s);
  if (lane == 0) out[row] = s;
}

__global__ void softcap_kernel(float* __restrict__ z, size_t n, float cap) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) z[i] = cap * tanhf(z[i] / cap);
}

__global__ void clear_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_softcap(float* z, size_t n, float cap, hipStream_t s) {
  softcap_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(z, n, cap);
  return hipGetLastError();
}

hipError_t launch_clear_u32(unsigned* p, int n, hipStream_t s) {
  clear_u32_kernel<<<(n + 255) / 256, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_ce_finalize(const float* partial, int nnb, const float* tgt_logit,
                              const int32_t* targets, const int32_t* tokens, int M, int V, float cap,
                              float* loss, unsigned* flags, hipStream_t s) {
  ce_finalize_kernel<<<(M + 3) / 4, 256, 0, s>>>(partial, nnb, tgt_logit, targets, tokens, M, V, cap,
                                                  loss, flags);
  return hipGetLastError();
}

hipError_t launch_prefix_target_logit(const void* x, const void* wu, const int32_t* targets, int M,
                                      int C, int c1, int V, float* out, hipStream_t s) {
  if (c1 % 8 || C % 8 || c1 > C) return hipErrorInvalidValue;
  prefix_target_logit_kernel<<<(M + 3) / 4, 256, 0, s>>>((const bf16*)x, (const bf16*)wu, targets, M, C,
                                                          c1, V, out);
  return hipGetLastError();
}

hipError_t launch_ce_mean(const float* loss, const int32_t* targets, int M, float* mean, hipStream_t s) {
  ce_mean_kernel<<<1, 1024, 0, s>>>(loss, targets, M, mean);
  return hipGetLastError();
}

}  // namespace gptk
