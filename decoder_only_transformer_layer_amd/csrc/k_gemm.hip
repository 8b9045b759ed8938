// GEMMs of the forward pass, C = A * B^T with A [M,K] and B [N,K] both K-contiguous (the
// row-major [out, in] weight layout), and fused epilogues:
//   STORE  - round to the activation type                    (QKV of the fp32 path)
//   RELU2  - max(0, c)^2, rounded                             (MLP up-projection)
//   RESID  - x += c into the fp32 residual stream             (attention out-proj, MLP down)
//   QKV    - q/k columns row-major, v columns transposed to [B][Hkv][D][T] (bf16 path)
//   CE     - softcap, per-row partial sum of exp(zhat - cap) per column block, and the target's
//            raw logit; the [M, V] logits are never written unless the caller asks for them
//            (then already softcapped).
//
// Sources: "The Mathematics of Karpathy's nanochat", sections "Causal Self-Attention"
// (projections, no bias), "Output Projection", "Feed-Forward Network (MLP)" (ReLU^2, 4x),
// "Logit Softcap" and "Cross-Entropy Loss".
//
// bf16 kernel (gfx950): v_mfma_f32_32x32x16_bf16 on 32x32 output tiles, fp32 accumulators.
// Block tile BM x BN x 64, WM x WN wavefronts each owning (BM/WM) x (BN/WN).  Operand tiles go
// global -> LDS directly (buffer loads with the LDS flag), double-buffered, one barrier per
// 64-wide K step.  LDS rows are 64 bf16 = eight 16-byte chunks; chunk c of row r lives at
// c ^ swz(r) so that the 16-byte fragment reads of 8 (or 16) consecutive rows hit distinct
// banks.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gptk {
namespace {

constexpr int BK = 64;
// Kernel-internal residual variants: + bf16 copy and row sums of squares; + next-layer mix.
constexpr int EPI_RESID_PROD = 5, EPI_RESID_MIX = 6;
template <int E> constexpr bool is_resid = E == EPI_RESID || E == EPI_RESID_PROD || E == EPI_RESID_MIX;
// Kernel-internal cross-entropy variant that also writes the raw logits (a separate kernel:
// the extra stores' addressing would otherwise cost the main loop registers).
constexpr int EPI_CE_LOGITS = 7;
// Kernel-internal cross-entropy variant that also evaluates the cross-entropy terms of the
// partial product over input columns [0, g.pre_k) (the nested model's kfront=1 logits) when the
// main loop reaches that K (see GemmArgs::partial1).
constexpr int EPI_CE_PREFIX = 8;
template <int E> constexpr bool is_ce = E == EPI_CE || E == EPI_CE_LOGITS || E == EPI_CE_PREFIX;

// s_waitcnt immediate waiting until at most n vector-memory operations are outstanding
// (gfx9 encoding: vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at bits 15:14; expcnt and lgkmcnt
// left at their maxima so they are not waited on).
constexpr int vmcnt_le(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
// s_waitcnt immediate waiting for all LDS/scalar-memory operations only.
constexpr int lgkmcnt_0 = 0xC07F;

__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }


// Block -> output tile.  Workgroups are dispatched round-robin over the 8 XCDs (each with its
// own L2), so block ids are first regrouped so that XCD x owns a contiguous 1/8 of the tile
// sequence; within it, tiles run down GM row-blocks before moving one column-block right, so
// the ~32 tiles resident on one XCD share a few A and B panels.
template <int GM>
__device__ __forceinline__ void tile_of(int pid, int nbm, int nbn, int& bm, int& bn) {
  const int nt = nbm * nbn;
  int t = pid;
  if ((nt & 7) == 0) t = (pid & 7) * (nt >> 3) + (pid >> 3);
  const int group = t / (GM * nbn);
  const int first = group * GM;
  const int gsz = min(nbm - first, GM);
  const int in = t - group * GM * nbn;
  bm = first + in % gsz;
  bn = in / gsz;
}

// The prefix's and the whole row's RMS scales from the per-slice sums of squares a residual
// producer wrote (slice-major, M per slice), in one pass over the row's slices: returns
// (1/sqrt(sum_{j < n1} ssp[j][row] / c1 + eps), 1/sqrt(sum_{j < n} ssp[j][row] / c + eps)).
// The row-sum order used everywhere: sixteen slices' loads in flight together, slice j below
// the largest multiple of 4 adds into s4[j % 4] and the rest into s4[0], each in increasing j,
// then (s4[0] + s4[1]) + (s4[2] + s4[3]).
__device__ __forceinline__ float2 row_rinv2(const float* ssp, int n1, float c1, int n, float c, float eps,
                                            int row, int M) {
  float s4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
  const int n4 = n & ~3, n14 = n1 & ~3;
  for (int j0 = 0; j0 < n; j0 += 16) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = j0 + u < n ? ssp[(size_t)(j0 + u) * M + row] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int j = j0 + u;
      if (j < n4) s4[u & 3] += v[u];
      else if (j < n) s4[0] += v[u];
      if (j < n14) p4[u & 3] += v[u];
      else if (j < n1) p4[0] += v[u];
    }
  }
  return make_float2(rsqrtf(((p4[0] + p4[1]) + (p4[2] + p4[3])) / c1 + eps),
                     rsqrtf(((s4[0] + s4[1]) + (s4[2] + s4[3])) / c + eps));
}

// RoPE-pair column order of a fused q|k tile of 384 columns (three 128-wide heads) on 64x192
// wavefront tiles: wavefront wn's fragments 2q and 2q+1 (32 columns each) hold, lane rl, the
// halves d = j and d = j + 64 of rotation pair P = 96 wn + 32 q + rl of the tile (head P / 64,
// j = P % 64).  Returns the tile-relative weight row (head * 128 + d) of tile column l.
__host__ __device__ __forceinline__ int qk_pair_row(int l) {
  const int wn = l / 192, f = (l % 192) / 32, r = l % 32;
  const int p = 96 * wn + 32 * (f >> 1) + r;
  return 128 * (p >> 6) + (p & 63) + 64 * (f & 1);
}

// One output tile (pid = its index in the GEMM's tile order) of C = A B^T with epilogue EPI.
// PRE: the tile may take a PrefixRMSNorm'd A as a two-part row scale (GemmArgs::pre_k); the
// kernel then holds BM more floats of LDS for the per-row factor.
template <int BM, int BN, int WM, int WN, int EPI, bool PRE = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int pid) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only types (buffer resources)
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  static_assert(FM * 32 == TM && FN * 32 == TN, "wave tile must be a multiple of 32");

  __shared__ __attribute__((aligned(16))) bf16 lds[2 * (BM + BN) * BK + (PRE ? 4 * BM : 0)];
  bf16* const As = lds;
  bf16* const Bs = lds + 2 * BM * BK;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int M = g.M, N = g.N, K = g.K;

  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  int bm, bn;
  tile_of<4>(pid, nbm, nbn, bm, bn);  // 4 row blocks per group: ~0.6-0.9 % faster than 8 or 16 at d24
  const int m0 = bm * BM, n0 = bn * BN;

  const bf16* const A = (const bf16*)g.A;
  const int lda = g.lda, ldb = g.ldb;
  const int nk = K / BK;

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

  // Direct global -> LDS loads (buffer_load_dwordx4 ... lds): one instruction per wave writes
  // 1 KB (8 rows of 64 bf16) of LDS at consecutive 16-byte slots, lane L filling slot L, so
  // each lane fetches the global chunk that the swizzled layout places at its slot.  The buffer
  // resource starts at the tile's first row and ends at the matrix's last row: rows past the
  // end read as zero, and the K offset travels in the scalar soffset.
  constexpr int NW = NT / 64;
  constexpr int AI = BM / 8 / NW, BI = BN / 8 / NW;  // 1 KB instructions per wave per operand
  static_assert(AI * NW * 8 == BM && BI * NW * 8 == BN, "direct-LDS tiling mismatch");
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (size_t)m0 * lda), (short)0, (int)min((size_t)(M - m0) * lda * 2, (size_t)0x7fffffff), 0x00020000);
  const int wids = __builtin_amdgcn_readfirstlane(wid);
  // B: each wave loads BN / NW consecutive rows of the tile, starting at row nw0.  Its resource
  // starts there, in the row segment (B0 | B1 | B2) that holds them: segment boundaries are
  // multiples of BN / NW rows, so a tile may straddle one while each wave's rows stay in one
  // segment.  Rows past the segment's end (past N in the last tile) read as zero.
  // Fused q|k tiles of the 64x192-wavefront layout (QKP) take their B rows in RoPE-pair order
  // instead: every 8-row block of the tile's LDS rows is 8 consecutive weight rows of the tile
  // (qk_pair_row), so the wave's resource starts at the tile's first row (the launcher keeps
  // q|k tiles inside one segment) and each block's row offset travels in the soffset.
  constexpr bool QKP = EPI == EPI_QKV && BN == 384 && WN == 2;
  bool perm = false;
  int nw0 = n0 + wids * BI * 8;
  int boff[QKP ? BI : 1];
  if constexpr (QKP) {
    perm = g.cs != nullptr && n0 < g.nqk;
    if (perm) nw0 = n0;
#pragma unroll
    for (int i = 0; i < BI; ++i) boff[i] = perm ? qk_pair_row((wids * BI + i) * 8) * ldb * 2 : i * 16 * ldb;
  }
  const bf16* Bseg;
  int nb0, nrows;
  if (nw0 < g.nseg0) { Bseg = (const bf16*)g.B0; nb0 = nw0; nrows = g.nseg0; }
  else if (nw0 < g.nseg0 + g.nseg1) { Bseg = (const bf16*)g.B1; nb0 = nw0 - g.nseg0; nrows = g.nseg1; }
  else { Bseg = (const bf16*)g.B2; nb0 = nw0 - g.nseg0 - g.nseg1; nrows = N - g.nseg0 - g.nseg1; }
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bseg + (size_t)(nb0 < nrows ? nb0 : 0) * ldb), (short)0,
      nb0 < nrows ? (int)min((size_t)(nrows - nb0) * ldb * 2, (size_t)0x7fffffff) : 0, 0x00020000);
  // Row block rb (8 rows) of an operand tile sits at row 8*rb: its lanes' chunk swizzle is
  // (lane & 7) ^ (lane >> 3) ^ (rb & 1), so two per-lane offsets serve every row block, and
  // the row block's start (relative to the wave's resource for B) and the K offset travel in
  // the scalar soffset.
  static_assert(AI % 2 == 0, "A row blocks per wave must be even");
  const int pb = (wids * BI) & 1;  // parity of this wave's first B row block (0 when BI is even)
  // The 256x384 tiles assume A and B share their row pitch (the launcher checks lda == ldb);
  // the other tiles keep a second offset pair for B.
  constexpr bool SAME_LD = BN == 384;
  int va[2], vb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = ((lane & 7) ^ (lane >> 3) ^ p) << 3;
    va[p] = ((lane >> 3) * lda + c) * 2;
    vb[p] = SAME_LD ? va[p] : ((lane >> 3) * ldb + c) * 2;
  }
  // The odd-BI tiles pick the B offset at run time: as named scalars (an array element selected
  // at run time can end up in scratch memory).
  const int vb0 = vb[0], vb1 = vb[1];
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
#define GEMM_ISSUE(buf, k0)                                                                   \
  do {                                                                                       \
    _Pragma("unroll") for (int i = 0; i < AI; ++i)                                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa,                                          \
        (lds_ptr_t)(As + (buf) * BM * BK + (wids * AI + i) * 512), 16, va[i & 1],           \
        (k0) * 2 + (wids * AI + i) * 16 * lda, 0, 0);                                        \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb,                                          \
        (lds_ptr_t)(Bs + (buf) * BN * BK + (wids * BI + i) * 512), 16,                      \
        (BI % 2 == 0 ? vb[i & 1] : (((pb + i) & 1) ? vb1 : vb0)),                            \
        (k0) * 2 + (QKP ? boff[QKP ? i : 0] : i * 16 * ldb), 0, 0);                         \
  } while (0)

  // Row-scale inputs staged early: a consumer of an un-normalised A (row scale from rs_ssp) has
  // the slice sums of its tile rows copied into LDS by DMA during the second-to-last K step, into
  // the buffer that step frees (the last step reads the other one), so the epilogue's row scale
  // reads LDS instead of waiting on memory.  Interior row blocks with at most 16 slices; not the
  // cross-entropy tiles (their epilogue holds too many registers already).
  constexpr bool SS_OK = !is_resid<EPI> && !is_ce<EPI>;
  const bool stage_ss = SS_OK && !PRE && g.rs_ssp != nullptr && nk >= 2 && g.rs_n <= 16 && m0 + BM <= M &&
                        (long)g.rs_n * M * 4 < 0x7fffffffL;
  const int ss_buf = nk & 1;  // the buffer the second-to-last K step frees
#define SS_ISSUE(buf)                                                                         \
  do {                                                                                       \
    const __amdgpu_buffer_rsrc_t rss = __builtin_amdgcn_make_buffer_rsrc(                    \
        (void*)(g.rs_ssp + m0), (short)0, (int)(((long)g.rs_n * M - m0) * 4), 0x00020000);   \
    for (int j = wids; j < g.rs_n; j += NT / 64)                                              \
      for (int q = 0; q < BM / 256; ++q)                                                      \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rss,                                         \
          (lds_ptr_t)((float*)(As + (buf) * BM * BK) + j * BM + q * 256), 16, lane * 16,      \
          (j * M + q * 256) * 4, 0, 0);                                                       \
  } while (0)

  // Software pipeline over 16-wide k-substeps with two fragment register sets: the reads for
  // substep s+1 are issued before the MFMAs of substep s.  The barrier that retires a K step's
  // buffer sits before that step's last 16 MFMAs, whose operands are already in registers, so
  // the barrier wait, the next tile's global->LDS issue and the first reads of the next K step
  // all overlap MFMA work.
  // ROLL (wide wave tiles, where two full fragment sets do not fit beside the accumulators):
  // A fragments keep two sets, B fragments one; a substep's MFMAs run B-fragment-major and each
  // B fragment is reloaded for the next substep right after its last MFMA, pinned in place.
  constexpr bool ROLL = FM * FN * 16 + 4 * 2 * (FM + FN) > 232;
  auto co_of = [&](int kk) { return ((2 * kk + hl) ^ sa) << 3; };
  auto rda = [&](const bf16* Ab, int kk, bf16x8 (&fa)[FM]) {
    const int co = co_of(kk);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) fa[fm] = *(const bf16x8*)(Ab + oa[fm] + co);
  };
  auto rdb = [&](const bf16* Bb, int kk, bf16x8 (&fb)[FN]) {
    const int co = co_of(kk);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) fb[fn] = *(const bf16x8*)(Bb + ob[fn] + co);
  };
  auto mm = [&](const bf16x8 (&fa)[FM], const bf16x8 (&fb)[FN]) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fm], fb[fn], acc[fm][fn], 0, 0, 0);
  };
  // PrefixRMSNorm'd A (nested models): the product over input columns [0, pre_k) carries the
  // prefix's scale 1/rms_p, the rest the whole row's 1/rms_a.  Once the K steps below pre_k are
  // done the accumulators are multiplied by pref[row] = (1/rms_p) / (1/rms_a); the epilogue's row
  // scale then applies 1/rms_a to the sum.
  // Thread i < BM owns tile row i: its (up to 16) slice sums are loaded with the first operand
  // tiles and summed when the main loop reaches pre_k, so their latency hides behind the first K
  // steps; then 1/rms_a goes where the epilogue's row scale reads it (the last BM floats of LDS).
  // More than 16 slices: computed before the main loop instead.
  float* const pref = (float*)(lds + 2 * (BM + BN) * BK);
  const int kpre = (PRE && g.pre_k > 0) ? g.pre_k / BK : -1;
  constexpr int PV = PRE ? 16 : 1;
  float pv[PV];
  const bool pv_held = PRE && kpre > 0 && g.rs_n <= 16;
  auto prefix_factors = [&]() {
    if constexpr (PRE) {
      if (kpre > 0) {
        float* const ra = (float*)lds + (sizeof(lds) / 4 - BM);
        if (pv_held) {
          const int row = m0 + tid;
#pragma unroll
          for (int u = 0; u < PV; ++u)
            pv[u] = (tid < BM && row < M && u < g.rs_n) ? g.rs_ssp[(size_t)u * M + row] : 0.f;
        } else {
          for (int i = tid; i < BM; i += NT) {
            const int row = m0 + i;
            const float2 r = row < M ? row_rinv2(g.rs_ssp, g.pre_n, g.pre_c, g.rs_n, g.rs_c, g.eps, row, M)
                                     : make_float2(0.f, 0.f);
            pref[i] = r.x / r.y;
            ra[i] = r.y;
          }
        }
      }
    }
  };
  // the held sums, in the row-sum order of row_rinv2 (slice j < n4 into s4[j % 4], the rest into s4[0])
  auto prefix_finish = [&]() {
    if constexpr (PRE) {
      if (pv_held) {
        float* const ra = (float*)lds + (sizeof(lds) / 4 - BM);
        if (tid < BM) {
          float s4[4] = {0.f, 0.f, 0.f, 0.f}, p4[4] = {0.f, 0.f, 0.f, 0.f};
          const int n4 = g.rs_n & ~3, n14 = g.pre_n & ~3;
#pragma unroll
          for (int u = 0; u < PV; ++u) {
            if (u < n4) s4[u & 3] += pv[u];
            else if (u < g.rs_n) s4[0] += pv[u];
            if (u < n14) p4[u & 3] += pv[u];
            else if (u < g.pre_n) p4[0] += pv[u];
          }
          const float rp = rsqrtf(((p4[0] + p4[1]) + (p4[2] + p4[3])) / g.pre_c + g.eps);
          const float rr = rsqrtf(((s4[0] + s4[1]) + (s4[2] + s4[3])) / g.rs_c + g.eps);
          pref[tid] = m0 + tid < M ? rp / rr : 0.f;
          ra[tid] = m0 + tid < M ? rr : 0.f;
        }
        __syncthreads();
      }
    }
  };
  auto prefix_rescale = [&]() {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 f = *(const f32x4*)(pref + wm * TM + fm * 32 + 8 * j + 4 * hl);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[fm][fn][4 * j + i] *= f[i];
      }
  };
  // EPI_CE_PREFIX: the cross-entropy terms of the partial product over columns [0, pre_k), per
  // row and wavefront (no LDS: the operand tiles occupy all of it), to partial1.
  auto prefix_ce = [&]() {
    if constexpr (EPI == EPI_CE_PREFIX) {
      const float k1 = 2.0f / g.cap * GPT_LOG2E, k2 = -2.0f * g.cap * GPT_LOG2E;
      const int cb = n0 + wn * TN + rl;
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const float q = rcp_fast(1.0f + exp2_fast(acc[fm][fn][r] * k1));
            sum += cb + fn * 32 < N ? exp2_fast(k2 * q) : 0.f;
          }
          sum = sum32(sum);
          const int row = m0 + wm * TM + fm * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (rl == 0 && row < M) g.partial1[(size_t)row * g.nnb1 + bn * WN + wn] = sum;
        }
    }
  };
  const int kce = EPI == EPI_CE_PREFIX ? g.pre_k / BK : -1;
  GEMM_ISSUE(0, 0);
  if (nk > 1) {
    GEMM_ISSUE(1, BK);
    prefix_factors();
    __builtin_amdgcn_s_waitcnt(vmcnt_le(AI + BI));
  } else {
    prefix_factors();
    __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
  }
  __syncthreads();
#define PIN __builtin_amdgcn_sched_barrier(0)
  // The K steps run as two loops with the same body: [0, ksplit) and [ksplit, nk), where ksplit
  // is the K step at which the prefix row scale or the prefix cross-entropy applies (nk if none),
  // so that the code between them stays out of the loops' register allocation.
  const int ksplit = kpre > 0 ? kpre : (kce > 0 ? kce : nk);
  auto at_split = [&]() {
    if constexpr (PRE) {
      if (kpre > 0) {
        prefix_finish();
        prefix_rescale();
      }
    }
    if constexpr (EPI == EPI_CE_PREFIX) {
      if (kce > 0) prefix_ce();
    }
  };
  if constexpr (!ROLL) {
    bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    rda(As, 0, fa0); rdb(Bs, 0, fb0);
    auto kstep = [&](int kt) {
      const int buf = kt & 1;
      const bf16* Ab = As + buf * BM * BK;
      const bf16* Bb = Bs + buf * BN * BK;
      PIN; rda(Ab, 1, fa1); rdb(Bb, 1, fb1); PIN; mm(fa0, fb0);
      PIN; rda(Ab, 2, fa0); rdb(Bb, 2, fb0); PIN; mm(fa1, fb1);
      PIN; rda(Ab, 3, fa1); rdb(Bb, 3, fb1); PIN; mm(fa0, fb0);
      PIN;
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));  // own loads of tile kt+1 have landed
      __syncthreads();                          // everyone's too; buffer `buf` fully read
      PIN;
      if (kt + 2 < nk) GEMM_ISSUE(buf, (kt + 2) * BK);
      else if (SS_OK && stage_ss && kt + 2 == nk) SS_ISSUE(buf);
      if (kt + 1 < nk) { rda(As + (buf ^ 1) * BM * BK, 0, fa0); rdb(Bs + (buf ^ 1) * BN * BK, 0, fb0); }
      PIN; mm(fa1, fb1);
      PIN;
      // The next substep-0 fragments were issued among those MFMAs; settling the LDS counter
      // here keeps the waitcnt pass from waiting on fresh reads at the loop top.
      __builtin_amdgcn_s_waitcnt(lgkmcnt_0);
    };
    if constexpr (PRE || EPI == EPI_CE_PREFIX) {
      for (int kt = 0; kt < ksplit; ++kt) kstep(kt);
      if (ksplit < nk) {
        at_split();
        for (int kt = ksplit; kt < nk; ++kt) kstep(kt);
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bf16* Ab = As + buf * BM * BK;
        const bf16* Bb = Bs + buf * BN * BK;
        PIN; rda(Ab, 1, fa1); rdb(Bb, 1, fb1); PIN; mm(fa0, fb0);
        PIN; rda(Ab, 2, fa0); rdb(Bb, 2, fb0); PIN; mm(fa1, fb1);
        PIN; rda(Ab, 3, fa1); rdb(Bb, 3, fb1); PIN; mm(fa0, fb0);
        PIN;
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
        __syncthreads();
        PIN;
        if (kt + 2 < nk) GEMM_ISSUE(buf, (kt + 2) * BK);
      else if (SS_OK && stage_ss && kt + 2 == nk) SS_ISSUE(buf);
        if (kt + 1 < nk) { rda(As + (buf ^ 1) * BM * BK, 0, fa0); rdb(Bs + (buf ^ 1) * BN * BK, 0, fb0); }
        PIN; mm(fa1, fb1);
        PIN;
        __builtin_amdgcn_s_waitcnt(lgkmcnt_0);
      }
    }
  } else if constexpr (QKP) {
    // 64x192 wavefront tiles: one A and one B fragment set, each fragment refilled for the next
    // substep right after its last MFMA of this one (A fragment fm after its row of FN MFMAs, B
    // fragment fn after the last row's), so every refill has at least FN MFMAs before its use.
    static_assert(!PRE && EPI != EPI_CE_PREFIX, "fully rolled loop has no split K step");
    bf16x8 fa[FM], fb[FN];
    auto mmroll2 = [&](const bf16* An, const bf16* Bn, int kn) {
      const int co = co_of(kn);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fm], fb[fn], acc[fm][fn], 0, 0, 0);
          if (fm == FM - 1) {
            fb[fn] = *(const bf16x8*)(Bn + ob[fn] + co);
            PIN;
          }
        }
        fa[fm] = *(const bf16x8*)(An + oa[fm] + co);
        PIN;
      }
    };
    rda(As, 0, fa); rdb(Bs, 0, fb);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      const bf16* Ab = As + buf * BM * BK;
      const bf16* Bb = Bs + buf * BN * BK;
      PIN; mmroll2(Ab, Bb, 1); mmroll2(Ab, Bb, 2); mmroll2(Ab, Bb, 3);
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));  // own loads of tile kt+1 have landed
      __syncthreads();                          // everyone's too; buffer `buf` fully read
      PIN;
      if (kt + 2 < nk) GEMM_ISSUE(buf, (kt + 2) * BK);
      else if (SS_OK && stage_ss && kt + 2 == nk) SS_ISSUE(buf);
      PIN; mmroll2(As + (buf ^ 1) * BM * BK, Bs + (buf ^ 1) * BN * BK, 0);
      __builtin_amdgcn_s_waitcnt(lgkmcnt_0);
    }
  } else {
    bf16x8 fa0[FM], fa1[FM], fb[FN];
    // MFMAs of one substep with fragments fa and fb; B fragment fn is then refilled from
    // (Bn, kn).  After the last K step these refills read a stale buffer: harmless, unused.
    auto mmroll = [&](const bf16x8 (&fa)[FM], const bf16* Bn, int kn) {
      const int co = co_of(kn);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fm], fb[fn], acc[fm][fn], 0, 0, 0);
        fb[fn] = *(const bf16x8*)(Bn + ob[fn] + co);
        PIN;
      }
    };
    rda(As, 0, fa0); rdb(Bs, 0, fb);
    auto kstep = [&](int kt) {
      const int buf = kt & 1;
      const bf16* Ab = As + buf * BM * BK;
      const bf16* Bb = Bs + buf * BN * BK;
      PIN; rda(Ab, 1, fa1); PIN; mmroll(fa0, Bb, 1);
      rda(Ab, 2, fa0); PIN; mmroll(fa1, Bb, 2);
      rda(Ab, 3, fa1); PIN; mmroll(fa0, Bb, 3);
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));  // own loads of tile kt+1 have landed
      __syncthreads();                          // everyone's too; buffer `buf` fully read
      PIN;
      if (kt + 2 < nk) GEMM_ISSUE(buf, (kt + 2) * BK);
      else if (SS_OK && stage_ss && kt + 2 == nk) SS_ISSUE(buf);
      rda(As + (buf ^ 1) * BM * BK, 0, fa0);
      PIN; mmroll(fa1, Bs + (buf ^ 1) * BN * BK, 0);
      __builtin_amdgcn_s_waitcnt(lgkmcnt_0);
    };
    if constexpr (PRE || EPI == EPI_CE_PREFIX) {
      for (int kt = 0; kt < ksplit; ++kt) kstep(kt);
      if (ksplit < nk) {
        at_split();
        for (int kt = ksplit; kt < nk; ++kt) kstep(kt);
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        const bf16* Ab = As + buf * BM * BK;
        const bf16* Bb = Bs + buf * BN * BK;
        PIN; rda(Ab, 1, fa1); PIN; mmroll(fa0, Bb, 1);
        rda(Ab, 2, fa0); PIN; mmroll(fa1, Bb, 2);
        rda(Ab, 3, fa1); PIN; mmroll(fa0, Bb, 3);
        __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
        __syncthreads();
        PIN;
        if (kt + 2 < nk) GEMM_ISSUE(buf, (kt + 2) * BK);
      else if (SS_OK && stage_ss && kt + 2 == nk) SS_ISSUE(buf);
        rda(As + (buf ^ 1) * BM * BK, 0, fa0);
        PIN; mmroll(fa1, Bs + (buf ^ 1) * BN * BK, 0);
        __builtin_amdgcn_s_waitcnt(lgkmcnt_0);
      }
    }
  }
#undef PIN
#undef GEMM_ISSUE
#undef SS_ISSUE

  // ---------------------------------------------------------------- epilogues
  // acc[fm][fn][r] is C[row][col] with row = m0 + wm*TM + fm*32 + 8*(r/4) + 4*hl + r%4 and
  // col = n0 + wn*TN + fn*32 + rl.  Interior tiles take a branch-free path so that all global
  // accesses of a lane can be in flight together.
  const int rbase = m0 + wm * TM + 4 * hl;
  const int cbase = n0 + wn * TN + rl;
  const bool interior = (m0 + BM <= M) && (n0 + BN <= N);

  if constexpr (!is_resid<EPI>) {
    if (g.rs_ssp != nullptr) {
      // A was not normalised: scale each output row by 1/rms of its A row, from the producer's
      // per-slice sums of squares (summed here in a fixed order).
      float* rinv = (float*)lds + (sizeof(lds) / 4 - BM);  // past any epilogue staging
      __syncthreads();  // every wavefront is done with the operand tiles
      // slices are stored slice-major ([slice][M]): consecutive threads read consecutive rows
      // (a prefix-scaled tile has its 1/rms_a there already)
      if (kpre <= 0 && stage_ss) {
        // the slice sums staged in LDS by SS_ISSUE, summed in row_rinv2's row-sum order
        const float* ssl = (const float*)(As + ss_buf * BM * BK);
        for (int i = tid; i < BM; i += NT) {
          float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;  // named: a run-time-indexed array would live in scratch
          const int n4 = g.rs_n & ~3;
          for (int j = 0; j < n4; j += 4) {
            s0 += ssl[j * BM + i];
            s1 += ssl[(j + 1) * BM + i];
            s2 += ssl[(j + 2) * BM + i];
            s3 += ssl[(j + 3) * BM + i];
          }
          for (int j = n4; j < g.rs_n; ++j) s0 += ssl[j * BM + i];
          rinv[i] = rsqrtf(((s0 + s1) + (s2 + s3)) / g.rs_c + g.eps);
        }
      } else if (kpre <= 0) for (int i = tid; i < BM; i += NT) {
        const int row = m0 + i;
        // Sixteen slices' loads are in flight together; slice j < n4 adds into s4[j % 4] and the
        // rest into s4[0], each in increasing j (row_rinv2's row-sum order).
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
        if (row < M) {
          const int n4 = g.rs_n & ~3;
          for (int j0 = 0; j0 < g.rs_n; j0 += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = j0 + u < g.rs_n ? g.rs_ssp[(size_t)(j0 + u) * M + row] : 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              if (j0 + u < n4) s4[u & 3] += v[u];
              else if (j0 + u < g.rs_n) s4[0] += v[u];
            }
          }
        }
        rinv[i] = rsqrtf(((s4[0] + s4[1]) + (s4[2] + s4[3])) / g.rs_c + g.eps);
      }
      __syncthreads();
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float sc = rinv[wm * TM + fm * 32 + 8 * (r >> 2) + 4 * hl + (r & 3)];
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) acc[fm][fn][r] *= sc;
        }
    }
  }

  if constexpr (EPI == EPI_STORE || EPI == EPI_RELU2) {
    bf16* const out = (bf16*)g.out;
    constexpr int LDP = TN + 4;  // staging row pitch (floats)
    if constexpr (WM * WN * 32 * LDP * 4 + BM * 4 <= (int)sizeof(lds)) {
      // Each 32-row group of the wavefront's tile is staged through LDS (wavefront-private,
      // fp32) and read back row-contiguous: every lane then stores 8 bf16 (16 bytes).
      constexpr int CPR = TN / 8, PER = CPR / 2;  // 16-byte chunks per row; per lane
      float* const stg = (float*)lds + wid * 32 * LDP;
      const bool vec = (g.ldo & 7) == 0;
      __syncthreads();  // every wavefront is done with the operand tiles
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float v = acc[fm][fn][r];
            if (EPI == EPI_RELU2) { v = fmaxf(v, 0.f); v = v * v; }
            stg[(8 * (r >> 2) + 4 * hl + (r & 3)) * LDP + fn * 32 + rl] = v;
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int idx = lane + 64 * k, lr = idx / CPR, ch = idx % CPR;
          const f32x4 a0 = *(const f32x4*)(stg + lr * LDP + ch * 8);
          const f32x4 a1 = *(const f32x4*)(stg + lr * LDP + ch * 8 + 4);
          bf16x8 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) { hv[e] = (bf16)a0[e]; hv[e + 4] = (bf16)a1[e]; }
          const int row = m0 + wm * TM + fm * 32 + lr, col = n0 + wn * TN + ch * 8;
          bf16* const op = out + (size_t)row * g.ldo + col;
          if ((interior || (row < M && col + 8 <= N)) && vec) {
            *(bf16x8*)op = hv;
          } else if (row < M) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < N) op[e] = hv[e];
          }
        }
        __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
      }
    } else {
      auto store = [&](auto checked) {
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
              if (!decltype(checked)::value || (row < M && col < N)) out[(size_t)row * g.ldo + col] = (bf16)v;
            }
          }
      };
      if (interior) store(std::false_type{}); else store(std::true_type{});
    }
  } else if constexpr (is_resid<EPI>) {
    // x += acc.  With a bf16 copy (the producer of the next RMSNorm) also: the optional
    // next-layer mix x = lam x + mu x0, the bf16 copy xb, and each row's sum of squares over
    // this wavefront's TN columns (one slice of width TN), written slice-major for the
    // consumer's row scale.  Each 32-row group of the wavefront's tile is staged through LDS
    // (wavefront-private) and read back row-contiguous, so that the global read-modify-write
    // moves 16 bytes per lane over whole 128-byte lines.
    constexpr bool prod = EPI != EPI_RESID, mix = EPI == EPI_RESID_MIX;
    constexpr int LDP = TN + 4;  // staging row pitch (floats)
    static_assert(WM * WN * 32 * LDP * 4 <= (int)sizeof(lds), "staging exceeds LDS");
    float* const out = (float*)g.out;
    float* const stg = (float*)lds + wid * 32 * LDP;
    const float lam = mix ? g.lam[g.layer] : 1.f, mu = mix ? g.mu[g.layer] : 0.f;
    const int slice = (g.col_off + n0 + wn * TN) / TN;
    const bool slice_live = prod && n0 + wn * TN < N;
    const bool vec = (g.ldo & 3) == 0;
    const int lr = lane >> 3, lc = (lane & 7) * 4;  // read-back: rows lr + 8j, columns lc + 32c
    __syncthreads();  // every wavefront is done with the operand tiles
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          stg[(8 * (r >> 2) + 4 * hl + (r & 3)) * LDP + fn * 32 + rl] = acc[fm][fn][r];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Row sum of squares of this lane's row over the wavefront's slice: 8-lane butterfly.
      auto put_ss = [&](int row, float ss) {
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        if ((lane & 7) == 0 && slice_live && row < M) g.ssp[(size_t)slice * M + row] = ss;
      };
      if (interior && vec) {
        // The x (and x0) chunks of the next 8 rows are loaded before this 8 rows' stores
        // are issued (the compiler cannot move a load of x past a store to x), so two row
        // groups' loads are in flight instead of one chunk's.
        f32x4 xv[2][FN], x0v[2][FN];
        auto prefetch = [&](int j) {
          const size_t ro = (size_t)(m0 + wm * TM + fm * 32 + lr + 8 * j) * g.ldo + n0 + wn * TN + lc;
#pragma unroll
          for (int c = 0; c < FN; ++c) {
            xv[j & 1][c] = *(const f32x4*)(out + ro + 32 * c);
            if (mix) x0v[j & 1][c] = *(const f32x4*)(g.x0 + ro + 32 * c);
          }
        };
        prefetch(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j + 1 < 4) prefetch(j + 1);
          const int row = m0 + wm * TM + fm * 32 + lr + 8 * j;
          const size_t ro = (size_t)row * g.ldo + n0 + wn * TN + lc;
          float ss = 0.f;
#pragma unroll
          for (int c = 0; c < FN; ++c) {
            const f32x4 a = *(const f32x4*)(stg + (lr + 8 * j) * LDP + 32 * c + lc);
            f32x4 v = xv[j & 1][c] + a;
            if (mix) v = lam * v + mu * x0v[j & 1][c];
            *(f32x4*)(out + ro + 32 * c) = v;
            if (prod) {
              bf16x4 h;
#pragma unroll
              for (int e = 0; e < 4; ++e) h[e] = (bf16)v[e];
              *(bf16x4*)(g.xb + ro + 32 * c) = h;
              ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
            }
          }
          if (prod) put_ss(row, ss);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = m0 + wm * TM + fm * 32 + lr + 8 * j;
          float ss = 0.f;
#pragma unroll
          for (int c = 0; c < FN; ++c) {
            const int col = n0 + wn * TN + 32 * c + lc;
            const f32x4 a = *(const f32x4*)(stg + (lr + 8 * j) * LDP + 32 * c + lc);
            const size_t o = (size_t)row * g.ldo + col;
            if (row < M && col + 4 <= N && vec) {
              f32x4 v = *(const f32x4*)(out + o) + a;
              if (mix) v = lam * v + mu * *(const f32x4*)(g.x0 + o);
              *(f32x4*)(out + o) = v;
              if (prod) {
                bf16x4 h;
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = (bf16)v[e];
                *(bf16x4*)(g.xb + o) = h;
                ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
              }
            } else if (row < M) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (col + e < N) {
                  float v = out[o + e] + a[e];
                  if (mix) v = lam * v + mu * g.x0[o + e];
                  out[o + e] = v;
                  if (prod) { g.xb[o + e] = (bf16)v; ss += v * v; }
                }
              }
            }
          }
          if (prod) put_ss(row, ss);
        }
      }
      __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
    }
  } else if constexpr (EPI == EPI_QKV && (TN == 96 || TN == 192)) {
    if constexpr (QKP) {
      if (perm) {
        // Fused q|k tile (head_dim 128) in RoPE-pair column order (qk_pair_row): the lane holds
        // both halves of each of its pairs, so RoPE is lane-local.  Heads 0 and 2 of the tile
        // lie in wavefronts 0 and 1; head 1's pairs j < 32 (wavefront 0, fragments 4-5) and
        // j >= 32 (wavefront 1, fragments 0-1) swap their squares through LDS.  Every head's sum
        // of squares is then formed as in the 128-wide form: the lane's pair j plus its pair
        // j + 32, then a 32-lane butterfly.  Output rows are staged 16 at a time through
        // wavefront-private LDS and written as 16-byte runs of q/k rows.
        bf16* qk = (bf16*)g.out;
        constexpr int LQ = TN + 8;                   // staging pitch (bf16)
        constexpr int STG = WM * WN * 16 * LQ * 2;   // staging bytes
        static_assert(STG + WM * WN * FM * 16 * 64 * 4 + BM * 4 <= (int)sizeof(lds), "q|k staging exceeds LDS");
        bf16* const stg = lds + wid * 16 * LQ;
        float* const xch = (float*)((char*)lds + STG);  // [wavefront][fm][r][lane] squares of head 1
        float* const xown = xch + wid * (FM * 16 * 64);
        const float* const xoth = xch + (wid ^ 1) * (FM * 16 * 64);  // the other wavefront of the row band
        const int qcol0 = n0 < g.nseg0 ? g.q_off + n0 : g.k_off + (n0 - g.nseg0);
        // Both phases are written for a compile-time wavefront column W (wn): pair q of it has
        // j = 32 * ((3 W + q) & 1) + rl; head 1 is its pair QM (fragments 4-5 for W = 0, 0-1 for
        // W = 1).  acc is only read: each phase rotates what it needs from the table.
        auto rope = [&](auto wc) {  // head 1's squares (after RoPE) to LDS
          constexpr int W = decltype(wc)::value, QM = W == 0 ? 2 : 0, PM = (3 * W + QM) & 1;
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            // the 32-row group is 32 consecutive positions of one sequence (T % 32 == 0)
            const float2* const csr = g.cs + ((m0 + wm * TM + fm * 32) % g.T + 4 * hl) * 64 + rl + PM * 32;
#pragma unroll
            for (int hc = 0; hc < 2; ++hc) {  // rows in chunks of 8: 8 table loads in flight
              float2 c[8];
#pragma unroll
              for (int q8 = 0; q8 < 8; ++q8) {
                const int r = 8 * hc + q8;
                c[q8] = csr[(8 * (r >> 2) + (r & 3)) * 64];
              }
#pragma unroll
              for (int q8 = 0; q8 < 8; ++q8) {
                const int r = 8 * hc + q8;
                const float u1 = acc[fm][2 * QM][r], u2 = acc[fm][2 * QM + 1][r];
                const float y1 = u1 * c[q8].x + u2 * c[q8].y, y2 = -u1 * c[q8].y + u2 * c[q8].x;
                xown[(fm * 16 + r) * 64 + lane] = y1 * y1 + y2 * y2;
              }
            }
          }
        };
        auto finish = [&](auto wc) {  // RoPE, norms, bf16 staging, 16-byte row stores
          constexpr int W = decltype(wc)::value, QA = W == 0 ? 0 : 1;  // whole head: pairs QA, QA + 1
#pragma unroll
          for (int fm = 0; fm < FM; ++fm) {
            const float2* const csr = g.cs + ((m0 + wm * TM + fm * 32) % g.T + 4 * hl) * 64 + rl;
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // rows 16h .. 16h+15 of the 32-row group
#pragma unroll
              for (int hc = 0; hc < 2; ++hc) {  // rows in chunks of 4: 8 table loads in flight
                float2 c[2][4];
#pragma unroll
                for (int q8 = 0; q8 < 4; ++q8) {
                  const int r = 8 * h + 4 * hc + q8;
#pragma unroll
                  for (int p = 0; p < 2; ++p) c[p][q8] = csr[(8 * (r >> 2) + (r & 3)) * 64 + p * 32];
                }
#pragma unroll
                for (int q8 = 0; q8 < 4; ++q8) {
                  const int r = 8 * h + 4 * hc + q8;
                  float y[6];
#pragma unroll
                  for (int q = 0; q < 3; ++q) {
                    const float2 cc = c[(3 * W + q) & 1][q8];
                    const float u1 = acc[fm][2 * q][r], u2 = acc[fm][2 * q + 1][r];
                    y[2 * q] = u1 * cc.x + u2 * cc.y;
                    y[2 * q + 1] = -u1 * cc.y + u2 * cc.x;
                  }
                  const float ea = y[2 * QA] * y[2 * QA] + y[2 * QA + 1] * y[2 * QA + 1];      // pairs j < 32
                  const float eb = y[2 * QA + 2] * y[2 * QA + 2] + y[2 * QA + 3] * y[2 * QA + 3];  // j >= 32
                  // head 1: wavefront 0 holds its pairs j < 32, wavefront 1 those j >= 32
                  const float em = xown[(fm * 16 + r) * 64 + lane], eo = xoth[(fm * 16 + r) * 64 + lane];
                  const float sw = rsqrtf(sum32(ea + eb) * (1.0f / 128.0f) + g.eps);
                  const float sm = rsqrtf(sum32(em + eo) * (1.0f / 128.0f) + g.eps);
                  bf16* const sr = stg + (8 * ((r >> 2) - 2 * h) + 4 * hl + (r & 3)) * LQ + rl;
#pragma unroll
                  for (int fn = 0; fn < FN; ++fn) {
                    const bool mid = W == 0 ? fn >= 4 : fn < 2;
                    sr[fn * 32] = (bf16)(y[fn] * (mid ? sm : sw));
                  }
                }
              }
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
              __builtin_amdgcn_wave_barrier();
              __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
              const int row0 = m0 + wm * TM + fm * 32 + 16 * h;
#pragma unroll
              for (int k = 0; k < 16 * (TN / 8) / 64; ++k) {  // 16 rows x 24 runs of 8 columns
                const int idx = lane + 64 * k, lr = idx / (TN / 8), ch = idx % (TN / 8);
                const int fn = ch >> 2, p0 = 96 * W + 32 * (fn >> 1);
                const int col = qcol0 + 128 * (p0 >> 6) + (p0 & 63) + 64 * (fn & 1) + 8 * (ch & 3);
                if (row0 + lr < M)
                  *(bf16x8*)(qk + (size_t)(row0 + lr) * g.ldo + col) = *(const bf16x8*)(stg + lr * LQ + 8 * ch);
              }
              __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
            }
          }
        };
        __syncthreads();  // every wavefront is done with the operand tiles
        if (wn == 0) rope(std::integral_constant<int, 0>{}); else rope(std::integral_constant<int, 1>{});
        __syncthreads();  // head 1's squares of both wavefronts are in LDS
        if (wn == 0) finish(std::integral_constant<int, 0>{}); else finish(std::integral_constant<int, 1>{});
        return;
      }
    }
    // v tiles (columns >= nqk, no value embeddings): the wavefront's tile is staged through
    // wavefront-private LDS transposed ([col][t], bf16) and written as 16-byte runs of 8
    // positions of v^T [B][Hkv][D][T].  64-row wavefront tiles stage both 32-row groups
    // together (in column groups of FG fragments, as LDS allows), so that each column's 64
    // positions go out as one 128-byte run (two where the rows cross into the next sequence);
    // 32-row wavefront tiles stage each group on its own.
    bf16* vt = (bf16*)g.vt;
    if constexpr (FM == 2) {
      constexpr int LV2 = 64 + 8;  // staging pitch (bf16)
      constexpr int FG = (WM * WN * FN * 32 * LV2 * 2 <= (int)sizeof(lds)) ? FN : FN / 2;
      static_assert(FN % FG == 0 && WM * WN * FG * 32 * LV2 * 2 <= (int)sizeof(lds), "v staging exceeds LDS");
      bf16* const stg = lds + wid * FG * 32 * LV2;
      __syncthreads();  // every wavefront is done with the operand tiles
      // the 64 rows are consecutive positions of one sequence, or of two (T % 32 == 0)
      const int row0 = m0 + wm * TM;
      const int bb0 = row0 / g.T, t00 = row0 - bb0 * g.T;
#pragma unroll
      for (int f0 = 0; f0 < FN; f0 += FG) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int f = 0; f < FG; ++f)
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // rows 32 fm + 8j + 4hl + (0..3): four consecutive t
              bf16x4 v4;
#pragma unroll
              for (int i = 0; i < 4; ++i) v4[i] = (bf16)acc[fm][f0 + f][4 * j + i];
              *(bf16x4*)(stg + (f * 32 + rl) * LV2 + 32 * fm + 8 * j + 4 * hl) = v4;
            }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int k = 0; k < FG * 32 * 8 / 64; ++k) {  // FG*32 columns x 8 runs of 8 positions
          const int idx = lane + 64 * k, cl = idx >> 3, ch = idx & 7;
          const int col = n0 + wn * TN + f0 * 32 + cl;
          if (col < N && row0 + ch * 8 < M) {
            const int vc = col - g.nqk, gg = g.v_head_off + vc / g.D, d = vc - (vc / g.D) * g.D;
            const bool nxt = t00 + ch * 8 >= g.T;  // these 8 rows begin the next sequence
            const int bb = bb0 + nxt, t = t00 + ch * 8 - (nxt ? g.T : 0);
            *(bf16x8*)(vt + ((size_t)(bb * g.Hkv + gg) * g.D + d) * g.T + t) =
                *(const bf16x8*)(stg + cl * LV2 + ch * 8);
          }
        }
        __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
      }
      return;
    }
    constexpr int LV = 32 + 8;  // staging pitch (bf16)
    static_assert(WM * WN * TN * LV * 2 <= (int)sizeof(lds), "v staging exceeds LDS");
    bf16* const stg = lds + wid * TN * LV;
    __syncthreads();  // every wavefront is done with the operand tiles
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // rows 8j + 4hl + (0..3): four consecutive t
          bf16x4 v4;
#pragma unroll
          for (int i = 0; i < 4; ++i) v4[i] = (bf16)acc[fm][fn][4 * j + i];
          *(bf16x4*)(stg + (fn * 32 + rl) * LV + 8 * j + 4 * hl) = v4;
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // 32 consecutive rows are 32 consecutive positions of one sequence (T % 32 == 0)
      const int row0 = m0 + wm * TM + fm * 32;
      const int bb = row0 / g.T, t0 = row0 - bb * g.T;
#pragma unroll
      for (int k = 0; k < TN * 4 / 64; ++k) {  // TN columns x 4 runs of 8 positions
        const int idx = lane + 64 * k, cl = idx >> 2, ch = idx & 3;
        const int col = n0 + wn * TN + cl;
        if (col < N && row0 + ch * 8 < M) {
          const int vc = col - g.nqk, gg = g.v_head_off + vc / g.D, d = vc - (vc / g.D) * g.D;
          *(bf16x8*)(vt + ((size_t)(bb * g.Hkv + gg) * g.D + d) * g.T + t0 + ch * 8) =
              *(const bf16x8*)(stg + cl * LV + ch * 8);
        }
      }
      __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
    }
  } else if constexpr (EPI == EPI_QKV) {
    bf16* qk = (bf16*)g.out;
    bf16* vt = (bf16*)g.vt;
    const int wcol0 = n0 + wn * TN;  // q, k and v segments are multiples of TN columns
    if constexpr (TN == 128) {
      if (g.cs != nullptr) {
        // This wavefront owns one whole 128-wide head (or two 64-wide ones) for its TM rows.  Each
        // 32-row group is finished in registers, staged through wavefront-private LDS as
        // bf16 and written back with 16-byte stores: q/k rows row-major, v transposed.
        // RoPE pairs (j, j+64) of a q/k head are tiles fn and fn+2 of the same lane; the
        // head's sum of squares is the lane's two pairs plus a 32-lane butterfly (the 32
        // lanes of a half share a row).  Rows go in chunks of 8 so that the 16 table loads of
        // a chunk are in flight together.
        constexpr int LQ = TN + 8, LV = 32 + 8;  // staging pitches (bf16): [row][col], [d][t]
        constexpr int WREG = 32 * LQ > TN * LV ? 32 * LQ : TN * LV;
        static_assert(WM * WN * WREG * 2 + BM * 4 <= (int)sizeof(lds), "QKV staging exceeds LDS");
        bf16* const stg = lds + wid * WREG;
        const bool live = wcol0 < N, is_qk = wcol0 < g.nqk;
        __syncthreads();  // every wavefront is done with the operand tiles
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
          if (is_qk && g.D == 64) {
            // two 64-wide heads: head h is tiles 2h and 2h+1, RoPE pairs (j, j+32) one lane's
            // tiles 2h, 2h+1, and each head's sum of squares its own 32-lane butterfly
#pragma unroll
            for (int hc = 0; hc < 2; ++hc) {
              float2 c[8];
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const int r = 8 * hc + q;
                const int t = (rbase + fm * 32 + 8 * (r >> 2) + (r & 3)) % g.T;
                c[q] = g.cs[t * 32 + rl];
              }
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const int r = 8 * hc + q;
                bf16* const sr = stg + (8 * (r >> 2) + 4 * hl + (r & 3)) * LQ + rl;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const float u1 = acc[fm][2 * h][r], u2 = acc[fm][2 * h + 1][r];
                  const float y1 = u1 * c[q].x + u2 * c[q].y, y2 = -u1 * c[q].y + u2 * c[q].x;
                  const float sc = rsqrtf(sum32(y1 * y1 + y2 * y2) * (1.0f / 64.0f) + g.eps);
                  sr[64 * h] = (bf16)(y1 * sc);
                  sr[64 * h + 32] = (bf16)(y2 * sc);
                }
              }
            }
          } else if (is_qk) {
#pragma unroll
            for (int hc = 0; hc < 2; ++hc) {
              float2 c[2][8];
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const int r = 8 * hc + q;
                const int t = (rbase + fm * 32 + 8 * (r >> 2) + (r & 3)) % g.T;
#pragma unroll
                for (int p = 0; p < 2; ++p) c[p][q] = g.cs[t * 64 + p * 32 + rl];
              }
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const int r = 8 * hc + q;
                float ss = 0.f;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                  const float u1 = acc[fm][p][r], u2 = acc[fm][p + 2][r];
                  const float y1 = u1 * c[p][q].x + u2 * c[p][q].y, y2 = -u1 * c[p][q].y + u2 * c[p][q].x;
                  acc[fm][p][r] = y1;
                  acc[fm][p + 2][r] = y2;
                  ss += y1 * y1 + y2 * y2;
                }
                const float sc = rsqrtf(sum32(ss) * (1.0f / 128.0f) + g.eps);
                bf16* const sr = stg + (8 * (r >> 2) + 4 * hl + (r & 3)) * LQ + rl;
#pragma unroll
                for (int fn = 0; fn < 4; ++fn) sr[fn * 32] = (bf16)(acc[fm][fn][r] * sc);
              }
            }
          } else {
            if (g.ve != nullptr) {
              // Value embedding: lane L's gate is row L % 32 of this group's; each lane then
              // adds g * ve[token] for its 16 rows and 4 columns.
              const int gg = g.v_head_off + (wcol0 - g.nqk) / g.D, ldve = g.Hkv * g.D;
              const int grp0 = m0 + wm * TM + fm * 32;
              const int lrow = lane & 31;
              float logit = 0.f;
              if (grp0 + lrow < M) {
                const bf16* xa = (const bf16*)g.A + (size_t)(grp0 + lrow) * g.lda;
                const bf16* wg = g.ve_gate + gg * 12;
#pragma unroll
                for (int c = 0; c < 12; ++c) logit += (float)xa[c] * (float)wg[c];
                if (g.rs_ssp != nullptr) logit *= ((const float*)lds)[sizeof(lds) / 4 - BM + wm * TM + fm * 32 + lrow];
              }
              const float gate = 3.f / (1.f + __expf(-logit));
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int lr = 8 * (r >> 2) + 4 * hl + (r & 3);
                const float gr = __shfl(gate, lr, 64);
                if (grp0 + lr < M) {
                  int tk = g.tokens[grp0 + lr];
                  tk = (tk >= 0 && tk < g.vocab) ? tk : 0;
                  const bf16* er = g.ve + (size_t)tk * ldve + gg * g.D + rl;
#pragma unroll
                  for (int fn = 0; fn < FN; ++fn) acc[fm][fn][r] += gr * (float)er[fn * 32];
                }
              }
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
              for (int j = 0; j < 4; ++j) {  // rows 8j + 4hl + (0..3): four consecutive t
                bf16x4 v4;
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = (bf16)acc[fm][fn][4 * j + i];
                *(bf16x4*)(stg + (fn * 32 + rl) * LV + 8 * j + 4 * hl) = v4;
              }
          }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int row0 = m0 + wm * TM + fm * 32;
          if (live && is_qk) {
            const int qc = wcol0 < g.nseg0 ? g.q_off + wcol0 : g.k_off + (wcol0 - g.nseg0);
#pragma unroll
            for (int k = 0; k < 8; ++k) {  // 32 rows x 16 chunks
              const int idx = lane + 64 * k, lr = idx >> 4, ch = idx & 15;
              if (row0 + lr < M)
                *(bf16x8*)(qk + (size_t)(row0 + lr) * g.ldo + qc + ch * 8) = *(const bf16x8*)(stg + lr * LQ + ch * 8);
            }
          } else if (live) {
            // 32 consecutive rows are 32 consecutive positions of one sequence (T % 32 == 0)
            const int bb = row0 / g.T, t0 = row0 - bb * g.T, gg = g.v_head_off + (wcol0 - g.nqk) / g.D;
            bf16* const vb = vt + ((size_t)(bb * g.Hkv + gg) * g.D) * g.T + t0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {  // 128 d rows x 4 chunks of 8 positions
              const int idx = lane + 64 * k, d = idx >> 2, ch = idx & 3;
              if (row0 + ch * 8 < M)
                *(bf16x8*)(vb + (size_t)d * g.T + ch * 8) = *(const bf16x8*)(stg + d * LV + ch * 8);
            }
          }
          __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
        }
        return;
      }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = cbase + fn * 32;
      if (col >= N) continue;
      if (col < g.nqk) {
        const int qcol = col < g.nseg0 ? g.q_off + col : g.k_off + (col - g.nseg0);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rbase + fm * 32 + 8 * (r >> 2) + (r & 3);
            if (row < M) qk[(size_t)row * g.ldo + qcol] = (bf16)acc[fm][fn][r];
          }
      } else {
        const int vc = col - g.nqk, gl = vc / g.D, d = vc - gl * g.D, gg = g.v_head_off + gl;
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
  } else if constexpr (is_ce<EPI>) {
    // Per row: sum over this block's columns of exp(zhat - cap).  Each lane sums its FN
    // columns, a 32-lane butterfly sums a wavefront's TN columns, and the WN wavefronts that
    // share a row combine through LDS (free after the main loop's final barrier).  Targets of
    // the block's rows are staged in LDS so that the target-logit pick-up is a predicated store.
    // With q = 1 / (1 + exp(2z / cap)): zhat = cap (1 - 2q) and exp(zhat - cap) = exp(-2 cap q),
    // the latter without the cancellation of subtracting cap from zhat.
    // EPI_CE_LOGITS also writes zhat: each 32-row group of the wavefront's tile is staged in LDS
    // past red and tgt and written back row-contiguous, 16 bytes per lane.
    constexpr bool LOGITS = EPI == EPI_CE_LOGITS;
    float* red = (float*)lds;                    // [BM][WN]
    int* tgt = (int*)(lds) + BM * WN;            // [BM]
    constexpr int LDP = TN + 4, STG0 = (BM * WN + BM + 63) / 64 * 64;  // staging pitch, offset (floats)
    static_assert(!LOGITS || (STG0 + WM * WN * 32 * LDP) * 4 <= (int)sizeof(lds), "logits staging exceeds LDS");
    float* const stg = (float*)lds + STG0 + wid * 32 * LDP;
    const float cap = g.cap;
    const float k1 = 2.0f / cap * GPT_LOG2E, k2 = -2.0f * cap * GPT_LOG2E;
    for (int i = tid; i < BM; i += NT) tgt[i] = (g.targets != nullptr && m0 + i < M) ? g.targets[m0 + i] : -1;
    __syncthreads();
    auto ce = [&](auto checked) {
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rloc = wm * TM + fm * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const int ycol = tgt[rloc] - cbase;    // target column relative to this lane's first
          float s = 0.f;
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const float z = acc[fm][fn][r];
            const float q = rcp_fast(1.0f + exp2_fast(z * k1));
            s += (!decltype(checked)::value || cbase + fn * 32 < N) ? exp2_fast(k2 * q) : 0.f;
            // raw logit; the loss kernel applies the softcap to it
            if (ycol == fn * 32) g.tgt_logit[m0 + rloc] = z;
            if constexpr (LOGITS) stg[(8 * (r >> 2) + 4 * hl + (r & 3)) * LDP + fn * 32 + rl] = cap - 2.0f * cap * q;
          }
          s = sum32(s);
          if (rl == 0) red[rloc * WN + wn] = s;
        }
        if constexpr (LOGITS) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          constexpr int CPR = TN / 4;  // 4-float chunks per staged row
          const bool vec = (N & 3) == 0;
#pragma unroll
          for (int k = 0; k < 32 * CPR / 64; ++k) {
            const int idx = lane + 64 * k, lr = idx / CPR, ch = idx % CPR;
            const int row = m0 + wm * TM + fm * 32 + lr, col = n0 + wn * TN + ch * 4;
            if (row < M) {
              const f32x4 v = *(const f32x4*)(stg + lr * LDP + ch * 4);
              float* const op = g.logits + (size_t)row * N + col;
              if (vec && col + 4 <= N) {
                *(f32x4*)op = v;
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (col + e < N) op[e] = v[e];
              }
            }
          }
          __builtin_amdgcn_wave_barrier();  // reads of this group precede the next group's writes
        }
      }
    };
    if (interior) ce(std::false_type{}); else ce(std::true_type{});
    __syncthreads();
    for (int rloc = tid; rloc < BM; rloc += NT) {
      const int row = m0 + rloc;
      if (row < M) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < WN; ++j) s += red[rloc * WN + j];
        g.partial[(size_t)row * g.nnb + bn] = s;
      }
    }
  }
#endif
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_bf16_kernel(GemmArgs g) {
  gemm_tile<BM, BN, WM, WN, EPI>(g, blockIdx.x);
}

// Two independent GEMMs with the same tile shape and epilogue in one launch: blocks
// [0, nb1) are the tiles of g1, the rest those of g2.  Blocks are dispatched in order, so g1
// is the one with the longer K and g2's shorter tiles fill in behind it.  PRE: either may take a
// PrefixRMSNorm'd A (GemmArgs::pre_k).
template <int BM, int BN, int WM, int WN, int EPI, bool PRE>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_bf16_pair_kernel(GemmArgs g1, GemmArgs g2, int nb1) {
  if ((int)blockIdx.x < nb1) gemm_tile<BM, BN, WM, WN, EPI, PRE>(g1, blockIdx.x);
  else gemm_tile<BM, BN, WM, WN, EPI, PRE>(g2, (int)blockIdx.x - nb1);
}

template <int BM, int BN, int WM, int WN>
hipError_t run_bf16(Epi epi, const GemmArgs& a, hipStream_t s) {
  const int grid = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  constexpr int NT = WM * WN * 64;
  switch (epi) {
    case EPI_STORE: GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_STORE>), grid, NT, s, a); break;
    case EPI_RELU2: GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_RELU2>), grid, NT, s, a); break;
    case EPI_RESID:
      if constexpr (WM * WN * 32 * (BN / WN + 4) * 4 > 2 * (BM + BN) * BK * 2) return hipErrorInvalidValue;  // staging would not fit
      else if (a.xb == nullptr) GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_RESID>), grid, NT, s, a);
      else if (a.lam == nullptr) GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_RESID_PROD>), grid, NT, s, a);
      else GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_RESID_MIX>), grid, NT, s, a);
      break;
    case EPI_QKV:
      // the tile plan gives this epilogue 256-wide or 128-wide tiles, and 384-wide ones to
      // launches of v columns only (no value embeddings)
      if constexpr (BN == 384) {
        if (a.nqk != 0 || a.ve != nullptr || a.T % 32) return hipErrorInvalidValue;
        GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_QKV>), grid, NT, s, a);
      } else if constexpr (BN != 256 && BN != 128) {
        return hipErrorInvalidValue;
      } else {
        GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_QKV>), grid, NT, s, a);
      }
      break;
    case EPI_CE:
      // 384-wide blocks only (the partial-sum layout has one column per block): 256-row tiles
      // for the loss alone, 128-row tiles when the logits are written too
      if constexpr (BN != 384) {
        return hipErrorInvalidValue;
      } else if constexpr (BM == 256) {
        if (a.logits != nullptr) return hipErrorInvalidValue;
        if (a.partial1 != nullptr) GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_CE_PREFIX>), grid, NT, s, a);
        else GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_CE>), grid, NT, s, a);
      } else {
        if (a.logits == nullptr) return hipErrorInvalidValue;
        GPTK_LAUNCH((gemm_bf16_kernel<BM, BN, WM, WN, EPI_CE_LOGITS>), grid, NT, s, a);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, bool PRE>
hipError_t run_bf16_pair_pre(Epi epi, const GemmArgs& a, const GemmArgs& b, hipStream_t s) {
  const int na = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int grid = na + ((b.M + BM - 1) / BM) * ((b.N + BN - 1) / BN);
  constexpr int NT = WM * WN * 64;
  if constexpr (WM > 2 && BN != 192) {  // tall 256/128-wide layouts: the fused q/k/v epilogue only
    if (epi != EPI_QKV) return hipErrorInvalidValue;
    GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_QKV, PRE>), grid, NT, s, a, b, na);
  } else if constexpr (PRE) {  // consumers of a PrefixRMSNorm'd input: ReLU^2 (MLP up) or q/k/v
    switch (epi) {
      case EPI_RELU2: GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_RELU2, PRE>), grid, NT, s, a, b, na); break;
      case EPI_QKV:
        if constexpr (BN == 192) return hipErrorInvalidValue;  // q/k/v take 256- or 128-wide tiles
        else GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_QKV, PRE>), grid, NT, s, a, b, na);
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (epi) {
      case EPI_STORE: GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_STORE, PRE>), grid, NT, s, a, b, na); break;
      case EPI_RELU2: GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_RELU2, PRE>), grid, NT, s, a, b, na); break;
      case EPI_RESID:
        if ((a.xb == nullptr) != (b.xb == nullptr) || (a.lam == nullptr) != (b.lam == nullptr))
          return hipErrorInvalidValue;  // both halves take the same residual variant
        if (a.xb == nullptr) GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_RESID, PRE>), grid, NT, s, a, b, na);
        else if (a.lam == nullptr) GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_RESID_PROD, PRE>), grid, NT, s, a, b, na);
        else GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_RESID_MIX, PRE>), grid, NT, s, a, b, na);
        break;
      case EPI_QKV:
        if constexpr (BN == 192) return hipErrorInvalidValue;  // q/k/v take 256- or 128-wide tiles
        else GPTK_LAUNCH((gemm_bf16_pair_kernel<BM, BN, WM, WN, EPI_QKV, PRE>), grid, NT, s, a, b, na);
        break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
hipError_t run_bf16_pair(Epi epi, const GemmArgs& a, const GemmArgs& b, hipStream_t s) {
  if (a.pre_k > 0 || b.pre_k > 0) return run_bf16_pair_pre<BM, BN, WM, WN, true>(epi, a, b, s);
  return run_bf16_pair_pre<BM, BN, WM, WN, false>(epi, a, b, s);
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

int gemm_f32_ce_blocks(int N) { return (N + FT - 1) / FT; }

namespace {

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

int gcd(int x, int y) { while (y) { const int t = x % y; x = y; y = t; } return x; }

// Columns [c0, N) of a GEMM as a GEMM of its own: the B row segments, the output pointer and
// the QKV column bookkeeping all shift by c0 (a multiple of 256).
GemmArgs shift_cols(const GemmArgs& a, Epi epi, int c0) {
  GemmArgs b = a;
  const void* seg[3] = {a.B0, a.B1, a.B2};
  const int start[3] = {0, a.nseg0, a.nseg0 + a.nseg1};
  const int len[3] = {a.nseg0, a.nseg1, a.N - a.nseg0 - a.nseg1};
  const void* nb[3] = {nullptr, nullptr, nullptr};
  int nl[3] = {0, 0, 0}, k = 0;
  for (int i = 0; i < 3; ++i) {
    const int s0 = start[i], s1 = start[i] + len[i];
    if (len[i] <= 0 || s1 <= c0) continue;
    const int off = c0 > s0 ? c0 - s0 : 0;
    nb[k] = (const bf16*)seg[i] + (size_t)off * a.ldb;
    nl[k] = s1 - (c0 > s0 ? c0 : s0);
    ++k;
  }
  b.N = a.N - c0;
  b.B0 = nb[0];
  b.B1 = k > 1 ? nb[1] : nb[0];
  b.B2 = k > 2 ? nb[2] : b.B1;
  b.nseg0 = nl[0];
  b.nseg1 = k > 1 ? nl[1] : 0;
  if (epi == EPI_RESID) {
    b.out = (float*)a.out + c0;
    if (a.xb) b.xb = a.xb + c0;
    if (a.x0) b.x0 = a.x0 + c0;
    b.col_off = a.col_off + c0;
  } else if (epi == EPI_QKV) {
    // the output base stays; the first remaining segment is addressed as the q segment and
    // is placed where it belonged (v columns are placed by head index)
    b.nqk = a.nqk - c0;
    if (c0 <= a.nseg0) b.q_off = a.q_off + c0;
    else if (c0 < a.nqk) b.q_off = a.k_off + (c0 - a.nseg0);
  } else {
    b.out = (bf16*)a.out + c0;
  }
  return b;
}

hipError_t run_main(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (epi == EPI_QKV && a.cs != nullptr) return run_bf16<256, 256, 4, 2>(epi, a, s);
  return run_bf16<256, 256, 2, 4>(epi, a, s);
}

hipError_t run_narrow(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (epi == EPI_QKV && a.cs != nullptr) {
    // fused q/k/v: eight wavefronts of 32x128 (whole heads), two per SIMD
    const int grid = ((a.M + 255) / 256) * ((a.N + 127) / 128);
    GPTK_LAUNCH((gemm_bf16_kernel<256, 128, 8, 1, EPI_QKV>), grid, 512, s, a);
    return hipGetLastError();
  }
  return run_bf16<256, 128, 2, 2>(epi, a, s);
}

// Interior column-segment boundaries (B0 | B1 | B2) must be multiples of `gran` columns.
bool seg_ok(const GemmArgs& a, int gran) {
  const int e0 = a.nseg0, e1 = a.nseg0 + a.nseg1;
  return (e0 >= a.N || e0 % gran == 0) && (e1 >= a.N || e1 % gran == 0);
}

// Granularity the 256x256 and 256x128 tiles need of segment boundaries: each wave's share of
// the B rows (32) lies in one segment, and with the fused q/k/v epilogue each wave's 128
// columns (whole heads) are all q, all k or all v.
int seg_gran(Epi epi, const GemmArgs& a) { return epi == EPI_QKV && a.cs != nullptr ? 128 : 32; }

// Tile plan of one GEMM.  Candidates: 256x384 tiles (8 wavefronts of 128x96) and 256x192
// tiles (8 wavefronts of 64x96) for the residual, ReLU^2 and store epilogues when N allows, and
// 256x256 tiles (8 wavefronts), the latter with the columns split when the tile count leaves a
// partial last round on the CUs: a leading part whose 256x256 tiles fill whole rounds and a
// tail of 256x128 tiles (8 wavefronts of 32x128 with the fused q/k/v epilogue, else 4 of
// 128x64), so the partial round costs half a tile per CU.
// Cost = rounds x tile area / relative efficiency (256x128 and 256x192 tiles run at about 3/4
// and 9/10 of the larger tiles' rate, their wavefront tiles re-reading LDS more per MFMA); the
// cheapest plan wins, wider tiles on a tie.  E.g. 16384 x 1536 takes one round of 256 tiles of
// 256x384 (256x256 would need 1.5 rounds) and 8192 x 1536 one round of 256 tiles of 256x192.
enum class Tiles { T256, T384, T192 };
struct Plan {
  Tiles tiles;
  int split_cols;  // 256x256 plan: columns of the leading part (0 = no split)
};

Plan plan_gemm(Epi epi, int M, int N, int nseg0, int nseg1, int ncu, bool same_ld = true) {
  auto seg_ok_n = [&](int bn) {
    const int e0 = nseg0, e1 = nseg0 + nseg1;
    return (e0 >= N || e0 % bn == 0) && (e1 >= N || e1 % bn == 0);
  };
  auto rounds = [&](long t) { return (double)((t + ncu - 1) / ncu); };
  const long nbm = (M + 255) / 256, nbn = (N + 255) / 256;
  const long tiles = nbm * nbn;
  Plan p{Tiles::T256, 0};
  double cost = rounds(tiles);  // in rounds of 256x256 tiles
  if (tiles > ncu && tiles % ncu != 0 && N % 256 == 0 && epi != EPI_CE) {
    const long per = ncu / gcd((int)nbm, ncu);  // column blocks per whole number of rounds
    const long c1 = (nbn / per) * per;
    if (c1 > 0 && c1 < nbn) {
      const double c = (double)(nbm * c1 / ncu) + rounds(nbm * (nbn - c1) * 2) * 0.5 / 0.75;
      if (c < cost) { cost = c; p.split_cols = (int)(c1 * 256); }
    }
  }
  if (epi == EPI_RESID || epi == EPI_RELU2 || epi == EPI_STORE) {
    if (N % 192 == 0 && seg_ok_n(192)) {
      const double c = rounds(nbm * (N / 192)) * 0.75 / 0.9;
      if (c <= cost) { cost = c; p = Plan{Tiles::T192, 0}; }
    }
    if (N % 384 == 0 && seg_ok_n(384) && same_ld) {
      const double c = rounds(nbm * (N / 384)) * 1.5;
      if (c <= cost) { cost = c; p = Plan{Tiles::T384, 0}; }
    }
  }
  return p;
}

}  // namespace

thread_local LaunchEvents launch_events;

int gemm_bf16_ce_blocks(int N) { return (N + 383) / 384; }

int gemm_resid_slice_cols(int M, int N) {
  return plan_gemm(EPI_RESID, M, N, N, 0, cu_count()).tiles == Tiles::T256 ? 64 : 96;
}

hipError_t launch_gemm_bf16(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.K % BK || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
  if (epi == EPI_CE) {  // 384-wide column blocks, as gemm_bf16_ce_blocks counts them
    if (a.lda != a.ldb) return hipErrorInvalidValue;
    if (a.partial1 != nullptr && (a.logits != nullptr || a.pre_k <= 0 || a.pre_k % BK || a.pre_k >= a.K ||
                                  a.nnb1 != 4 * a.nnb))
      return hipErrorInvalidValue;
    // Writing the logits too takes 128-row tiles: the staged stores' addressing would otherwise
    // push the 256-row tiles' main loop past the register file.
    return a.logits != nullptr ? run_bf16<128, 384, 2, 4>(epi, a, s) : run_bf16<256, 384, 2, 4>(epi, a, s);
  }
  if (epi == EPI_QKV && a.cs != nullptr && a.D != 128 && a.D != 64) return hipErrorInvalidValue;
  // Fused q/k/v with 128-wide heads whose q, k and v segments are multiples of 384 columns (three
  // heads): one launch of 256x384 tiles, eight wavefronts of 64x192, q|k tiles in RoPE-pair column
  // order (e.g. d24: 3 rounds of the CUs, against 3 of 256x256 q|k tiles plus 1 of v tiles).
  if (epi == EPI_QKV && a.cs != nullptr && a.D == 128 && a.ve == nullptr && a.lda == a.ldb && a.T % 32 == 0 &&
      a.nqk > 0 && a.nseg0 % 384 == 0 && a.nseg0 + a.nseg1 == a.nqk && a.nqk % 384 == 0 && a.N % 384 == 0 &&
      a.ldo % 8 == 0 && a.q_off % 8 == 0 && a.k_off % 8 == 0) {
    const int grid = ((a.M + 255) / 256) * (a.N / 384);
    GPTK_LAUNCH((gemm_bf16_kernel<256, 384, 4, 2, EPI_QKV>), grid, 512, s, a);
    return hipGetLastError();
  }
  // Fused q/k/v: the q and k columns as one GEMM (256-wide tiles, whole heads per wavefront) and
  // the v columns as another on 256x384 tiles when that takes fewer rounds of the CUs than one
  // plan for all columns (e.g. d24: 3 rounds of q|k + 1 of v, against 4.5 for the whole).
  if (epi == EPI_QKV && a.cs != nullptr && a.ve == nullptr && a.nqk > 0 && a.nqk < a.N &&
      a.nqk % 256 == 0 && (a.N - a.nqk) % 384 == 0 && a.T % 32 == 0 && a.lda == a.ldb &&
      seg_ok(a, seg_gran(epi, a))) {
    const int ncu = cu_count();
    auto cost = [&](const Plan& q, int n) {
      const long nbm = (a.M + 255) / 256, t = nbm * (n / 256);
      if (q.split_cols <= 0) return (double)((t + ncu - 1) / ncu);
      const long c1 = q.split_cols / 256;
      return (double)(nbm * c1 / ncu) + (double)((nbm * (n / 256 - c1) * 2 + ncu - 1) / ncu) * 0.5 / 0.75;
    };
    const Plan whole = plan_gemm(epi, a.M, a.N, a.nseg0, a.nseg1, ncu);
    const Plan qk = plan_gemm(epi, a.M, a.nqk, a.nseg0, a.nseg1, ncu);
    const long vt = (long)((a.M + 255) / 256) * ((a.N - a.nqk) / 384);
    const double c_split = cost(qk, a.nqk) + (double)((vt + ncu - 1) / ncu) * 1.5;
    if (whole.tiles == Tiles::T256 && qk.tiles == Tiles::T256 && c_split < cost(whole, a.N)) {
      GemmArgs h = a;
      h.N = a.nqk;
      hipError_t e;
      if (qk.split_cols > 0) {
        GemmArgs head = h;
        head.N = qk.split_cols;
        if (head.nseg0 > head.N) head.nseg0 = head.N;
        if (head.nseg0 + head.nseg1 > head.N) head.nseg1 = head.N - head.nseg0;
        e = run_main(epi, head, s);
        if (e == hipSuccess) e = run_narrow(epi, shift_cols(h, epi, qk.split_cols), s);
      } else {
        e = run_main(epi, h, s);
      }
      if (e != hipSuccess) return e;
      return run_bf16<256, 384, 2, 4>(epi, shift_cols(a, epi, a.nqk), s);
    }
  }
  const Plan p = plan_gemm(epi, a.M, a.N, a.nseg0, a.nseg1, cu_count(), a.lda == a.ldb);
  if (p.tiles == Tiles::T384) return run_bf16<256, 384, 2, 4>(epi, a, s);  // slices of 96 columns
  if (p.tiles == Tiles::T192) return run_bf16<256, 192, 4, 2>(epi, a, s);  // slices of 96 columns
  if (!seg_ok(a, seg_gran(epi, a))) return hipErrorInvalidValue;
  if (p.split_cols > 0) {  // both parts keep 64-column wavefront slices
    GemmArgs head = a;
    head.N = p.split_cols;
    if (head.nseg0 > head.N) head.nseg0 = head.N;
    if (head.nseg0 + head.nseg1 > head.N) head.nseg1 = head.N - head.nseg0;
    hipError_t e = run_main(epi, head, s);
    if (e != hipSuccess) return e;
    return run_narrow(epi, shift_cols(a, epi, p.split_cols), s);
  }
  return run_main(epi, a, s);
}

// Tile shape of a grouped pair (launch_gemm_bf16_pair): 256x192 tiles (wavefront tiles of 64x96)
// instead of 256x256 when that fills the CUs in fewer rounds, at ~0.9 of the larger tiles' rate:
// e.g. the nested model's MLP-down and out-projection pairs at M = 8192 make exactly 256 tiles
// of 256x192 against 224 of 256x256, whose longest ones then set the time.
enum class PairTiles { T192, T256, SEPARATE };
PairTiles plan_pair(Epi epi, const GemmArgs& a, const GemmArgs& b) {
  const bool fused = epi == EPI_QKV && (a.cs != nullptr || b.cs != nullptr);
  if (!fused && epi != EPI_QKV && a.N % 192 == 0 && b.N % 192 == 0 && seg_ok(a, 192) && seg_ok(b, 192)) {
    const int ncu = cu_count();
    auto rounds = [&](int bn) {
      const long t = (long)((a.M + 255) / 256) * ((a.N + bn - 1) / bn) + (long)((b.M + 255) / 256) * ((b.N + bn - 1) / bn);
      return (double)((t + ncu - 1) / ncu);
    };
    const double c256 = seg_ok(a, seg_gran(epi, a)) && seg_ok(b, seg_gran(epi, b)) ? rounds(256) : 1e30;
    if (rounds(192) * 0.75 / 0.9 < c256) return PairTiles::T192;
  }
  const int gran = fused ? 128 : 32;
  if (seg_ok(a, gran) && seg_ok(b, gran)) return PairTiles::T256;
  return PairTiles::SEPARATE;
}

hipError_t launch_gemm_bf16_pair(Epi epi, const GemmArgs& a, const GemmArgs& b, hipStream_t s) {
  if (a.N <= 0) return launch_gemm_bf16(epi, b, s);
  if (b.N <= 0) return launch_gemm_bf16(epi, a, s);
  if (a.K % BK || b.K % BK || a.M <= 0 || b.M <= 0 || epi == EPI_CE) return hipErrorInvalidValue;
  if ((a.pre_k > 0 && (a.pre_k % BK || a.rs_ssp == nullptr)) || (b.pre_k > 0 && (b.pre_k % BK || b.rs_ssp == nullptr)))
    return hipErrorInvalidValue;
  const bool fused = epi == EPI_QKV && (a.cs != nullptr || b.cs != nullptr);
  if (fused && (a.cs == nullptr || b.cs == nullptr || a.D != b.D || (a.D != 128 && a.D != 64)))
    return hipErrorInvalidValue;
  switch (plan_pair(epi, a, b)) {
    case PairTiles::T192: return run_bf16_pair<256, 192, 4, 2>(epi, a, b, s);
    case PairTiles::T256:
      return fused ? run_bf16_pair<256, 256, 4, 2>(epi, a, b, s) : run_bf16_pair<256, 256, 2, 4>(epi, a, b, s);
    default: break;
  }
  if (a.pre_k > 0 || b.pre_k > 0) return hipErrorInvalidValue;  // the single-GEMM tiles take no prefix scale
  const hipError_t e = launch_gemm_bf16(epi, a, s);
  return e != hipSuccess ? e : launch_gemm_bf16(epi, b, s);
}

int gemm_pair_resid_slice_cols(const GemmArgs& a, const GemmArgs& b) {
  switch (plan_pair(EPI_RESID, a, b)) {
    case PairTiles::T192: return 96;   // 4 x 2 wavefronts of 64 x 96
    case PairTiles::T256: return 64;   // 2 x 4 wavefronts of 128 x 64
    default: return 0;                 // launched separately: slices of each GEMM's own plan
  }
}

hipError_t launch_gemm_f32(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.K <= 0) return hipErrorInvalidValue;
  const int grid = ((a.M + FT - 1) / FT) * ((a.N + FT - 1) / FT);
  switch (epi) {
    case EPI_STORE: case EPI_QKV: GPTK_LAUNCH((gemm_f32_kernel<EPI_STORE>), grid, 256, s, a); break;
    case EPI_RELU2: GPTK_LAUNCH((gemm_f32_kernel<EPI_RELU2>), grid, 256, s, a); break;
    case EPI_RESID: GPTK_LAUNCH((gemm_f32_kernel<EPI_RESID>), grid, 256, s, a); break;
    case EPI_CE: GPTK_LAUNCH((gemm_f32_kernel<EPI_CE>), grid, 256, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gptk
