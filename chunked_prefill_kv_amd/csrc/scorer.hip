// K3: stream the history keys once and score them against the kept queries.
//   s_i = max_{t in S_h} g_t . k_i / |k_i|
// which is the max over kept tokens of the mean over the group's heads of the
// per-head cosines (g_t is the mean of the token's unit query heads).
// Sources: QUOKA paper summary (hw-hk.tistory.com/367), "Scoring via Cosine
// Similarity" and "Aggregation Across Queries and KV Groups" (max over the
// query axis, mean over the GQA axis, pre-aggregation); "QUOKA Explained",
// "Letting those queries score the history", "Why take the maximum".
//
// The epilogue also builds the first-level histogram of the top-B select
// (linear bins over [-1, 1]) so that the scores are not re-read for it.
//
// MODE selects the baselines' arithmetic (kModeDot: no division by |k_i|,
// histogram over all floats; kModeHeads: each kept token brings G unit head
// rows, summed per token before the max and divided by G). one_row: the
// query select laid out a single row (the mean-query baselines).
#include "common.h"
#include "internal.h"

namespace quoka {

// Adds the workgroup's score histogram to the problem's.
__device__ __forceinline__ void flush_hist(const uint32_t* lhist, uint32_t* __restrict__ hist,
                                           int prob) {
  uint32_t* gh = hist + (int64_t)prob * kScoreBins;
  for (int i = threadIdx.x; i < kScoreBins; i += 256) {
    const uint32_t c = lhist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// bf16 keys, MFMA v_mfma_f32_16x16x32_bf16.
//   A = kept queries [16 x 32 d] from LDS (pre-laid-out by the query select as
//       hi and lo bf16 terms of the fp32 g, so g ~ hi + lo to 2^-16),
//   B = keys [32 d x 16 keys] straight from global memory (each lane reads 16
//       contiguous bytes of one key row; 4 lanes cover 64 B of a row),
//   C = [16 queries x 16 keys]; lane l holds key column l%16, so the max over
//       queries is a per-lane max followed by two cross-lane steps.
// One workgroup = 4 waves = NB * 256 keys of one (sequence, KV head). Wave w
// scores the 64-key blocks w, w + 4, w + 8, ... of the tile; two blocks are
// in flight per wave, and the block just scored is refilled with the one two
// ahead. Keys are read through a buffer resource that covers exactly the
// tile's keys, so reads past its last key return zeros without a memory
// access. The block loop is unrolled at compile time and every load in it
// is unconditional (only the scoring of blocks past the sequence's end is
// skipped), so the compiler waits for exactly the 16 loads of the block in
// hand rather than for every load in flight.
template <int D, int NB, int MODE>
__global__ __launch_bounds__(256) void scorer_mfma_kernel(
    const bf16* __restrict__ k_hist, const int32_t* __restrict__ cu_chunk,
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int q_budget, int nq_pad, const bf16x8* __restrict__ gsel,
    float* __restrict__ scores, uint32_t* __restrict__ hist, int one_row, int G) {
  constexpr int score_keys = NB * 256;
  constexpr int NDS = D / 32;                 // d-steps per key
  const int GH = MODE == kModeHeads ? G : 1;  // rows per kept token
  const int blk = blockIdx.x, h = blockIdx.y;
  const int32_t* sb_off = plan + (S + 1);
  const int s = upper_seq(sb_off, S, blk);
  const int k_begin = (blk - sb_off[s]) * score_keys;
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int k_end = min(L, k_begin + score_keys);
  const int n = min(one_row ? 1 : q_budget, cu_chunk[s + 1] - cu_chunk[s]);
  const int nqb = (n + 15) / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int prob = s * Hkv + h;
  const int first = k_begin + wave * 64;  // this wave's first key

  // keys [k_begin, k_end) of this (sequence, head); row stride Hkv * D
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2u;
  const __amdgpu_buffer_rsrc_t rk =
      make_rsrc(k_hist + ((int64_t)(h_off + k_begin) * Hkv + h) * D,
                k_end > k_begin ? (uint32_t)(k_end - k_begin - 1) * row_bytes + D * 2u : 0u);
  const uint32_t lane_off = (uint32_t)(lane & 15) * row_bytes + (uint32_t)(lane >> 4) * 16u;
  auto load = [=](int j, bf16x8 (&b)[4][NDS]) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)(wave * 64 + j * 256);  // tile-relative
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        b[kb][ds] = buffer_load_bf16x8(rk, (k0 + kb * 16) * row_bytes + lane_off + ds * 64u);
  };
  // The kept-query rows are read (into registers) and stored to LDS before
  // any key is requested: requested after the keys, their reads wait behind
  // the whole key stream of the chip. Then the first two key blocks of every
  // wave go out together, so the stream has no gap between the rounds.
  extern __shared__ char smem[];
  uint32_t* lhist = (uint32_t*)smem;                       // kScoreBins
  bf16x8* lg = (bf16x8*)(smem + kScoreBins * 4);           // nqb * GH * NDS * 2 * 64
  const bf16x8* gsrc = gsel + (int64_t)prob * (nq_pad / 16) * GH * NDS * 2 * 64;
  const int nstage = nqb * GH * NDS * 2 * 64;
  constexpr int kStageU = 16;  // 16-byte pieces per thread staged through registers
  {
    bf16x8 stg[kStageU];
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int i = u * 256 + (int)threadIdx.x;
      if (i < nstage) stg[u] = gsrc[i];
    }
    for (int i = threadIdx.x; i < kScoreBins; i += 256) lhist[i] = 0u;
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int i = u * 256 + (int)threadIdx.x;
      if (i < nstage) lg[i] = stg[u];
    }
  }
  bf16x8 b0[4][NDS], b1[4][NDS];
  load(0, b0);
  if constexpr (NB > 1) load(1, b1);
  // Only the per-head rows outgrow the register staging (at most 128 rows of
  // d <= 128 otherwise); their rest is copied behind the first key loads.
  if constexpr (MODE == kModeHeads) {
    if (nstage > kStageU * 256)
      block_copy<256, 8>(lg + kStageU * 256, gsrc + kStageU * 256, nstage - kStageU * 256);
  }
  __syncthreads();

  float* srow = scores + (int64_t)h * TL + h_off;
  auto score = [=](int j, bf16x8 (&cur)[4][NDS]) __attribute__((always_inline)) {
    const int k0 = first + j * 256;
    float nsq[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int kb = 0; kb < 4 && MODE != kModeDot; ++kb) {
      // |k|^2 from bf16 pairs: two exact products per instruction, fp32 sums
      float ss = 0.f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 v = cur[kb][ds];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {v[e], v[e + 1]};
          ss = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, ss, false);
        }
      }
      ss = rows_sum(ss);
      nsq[kb] = ss;
    }
    float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int qb = 0; qb < nqb; ++qb) {
      f32x4 acc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int jh = 0; jh < GH; ++jh) {  // per head rows accumulate: the sum over heads
        const bf16x8* la = lg + (qb * GH + jh) * NDS * 2 * 64 + lane;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const bf16x8 ahi = la[(ds * 2 + 0) * 64];
          const bf16x8 alo = la[(ds * 2 + 1) * 64];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, cur[kb][ds], acc[kb], 0, 0, 0);
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, cur[kb][ds], acc[kb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        m[kb] = fmaxf(m[kb], fmaxf(fmaxf(acc[kb][0], acc[kb][1]), fmaxf(acc[kb][2], acc[kb][3])));
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      m[kb] = rows_max(m[kb]);
    }
    // lane l stores key k0 + l: its column is l%16 of key block l/16
    const int kb = lane >> 4;
    const float mm = kb == 0 ? m[0] : kb == 1 ? m[1] : kb == 2 ? m[2] : m[3];
    const float ns = kb == 0 ? nsq[0] : kb == 1 ? nsq[1] : kb == 2 ? nsq[2] : nsq[3];
    const int key = k0 + lane;
    if (key < k_end) {
      float sc;
      if constexpr (MODE == kModeDot) sc = n > 0 ? mm : 0.f;
      else if constexpr (MODE == kModeHeads) sc = (n > 0 && ns > 0.f) ? mm / ((float)G * sqrtf(ns)) : 0.f;
      else sc = (n > 0 && ns > 0.f) ? mm / sqrtf(ns) : 0.f;
      srow[key] = sc;
      atomicAdd(&lhist[MODE == kModeDot ? score_bin_raw(sc) : score_bin(sc)], 1u);
    }
  };
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    bf16x8 (&cur)[4][NDS] = (j & 1) ? b1 : b0;
    if (first + j * 256 < k_end) score(j, cur);
    if (j + 2 < NB) load(j + 2, cur);  // the block just scored is refilled two ahead
  }
  __syncthreads();
  flush_hist(lhist, hist, prob);
}

// fp32 keys (and any dtype as a reference path): one key per thread, kept
// queries as fp32 rows in LDS read by broadcast.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256) void scorer_valu_kernel(
    const T* __restrict__ k_hist, const int32_t* __restrict__ cu_chunk,
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int q_budget, int nq_pad, const float* __restrict__ gsel,
    float* __restrict__ scores, uint32_t* __restrict__ hist, int score_keys, int one_row, int G) {
  const int GH = MODE == kModeHeads ? G : 1;
  const int blk = blockIdx.x, h = blockIdx.y;
  const int32_t* sb_off = plan + (S + 1);
  const int s = upper_seq(sb_off, S, blk);
  const int k_begin = (blk - sb_off[s]) * score_keys;
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int k_end = min(L, k_begin + score_keys);
  const int n = min(one_row ? 1 : q_budget, cu_chunk[s + 1] - cu_chunk[s]);
  const int prob = s * Hkv + h;

  extern __shared__ char smem[];
  uint32_t* lhist = (uint32_t*)smem;
  float* lg = (float*)(smem + kScoreBins * 4);  // n x GH x D
  for (int i = threadIdx.x; i < kScoreBins; i += 256) lhist[i] = 0u;
  block_copy<256, 8>(lg, gsel + (int64_t)prob * nq_pad * GH * D, n * GH * D);
  __syncthreads();

  float* srow = scores + (int64_t)h * TL + h_off;
  for (int key = k_begin + threadIdx.x; key < k_end; key += 256) {
    const T* row = k_hist + ((int64_t)(h_off + key) * Hkv + h) * D;
    float k[D];
    float ss = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      k[d] = to_f32(row[d]);
      ss = fmaf(k[d], k[d], ss);
    }
    float m = -INFINITY;
    for (int r = 0; r < n; ++r) {
      float tot = 0.f;
      for (int j = 0; j < GH; ++j) {  // per head rows: the sum over heads
        const float* gr = lg + (r * GH + j) * D;
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(gr[d], k[d], dot);
        tot += dot;
      }
      m = fmaxf(m, tot);
    }
    float sc;
    if constexpr (MODE == kModeDot) sc = n > 0 ? m : 0.f;
    else if constexpr (MODE == kModeHeads) sc = (n > 0 && ss > 0.f) ? m / ((float)G * sqrtf(ss)) : 0.f;
    else sc = (n > 0 && ss > 0.f) ? m / sqrtf(ss) : 0.f;
    srow[key] = sc;
    atomicAdd(&lhist[MODE == kModeDot ? score_bin_raw(sc) : score_bin(sc)], 1u);
  }
  __syncthreads();
  flush_hist(lhist, hist, prob);
}

hipError_t set_scorer_lds_limit(int bytes, int bytes_heads) {
  const void* fns[] = {
#define QUOKA_SCORER_NB(D, M)                                                                 \
  (const void*)scorer_mfma_kernel<D, 1, M>, (const void*)scorer_mfma_kernel<D, 2, M>,         \
      (const void*)scorer_mfma_kernel<D, 4, M>, (const void*)scorer_mfma_kernel<D, 8, M>
      QUOKA_SCORER_NB(128, kModeCos), QUOKA_SCORER_NB(64, kModeCos),
      QUOKA_SCORER_NB(128, kModeDot), QUOKA_SCORER_NB(64, kModeDot),
      (const void*)scorer_valu_kernel<float, 128, kModeCos>,
      (const void*)scorer_valu_kernel<float, 64, kModeCos>,
      (const void*)scorer_valu_kernel<float, 128, kModeDot>,
      (const void*)scorer_valu_kernel<float, 64, kModeDot>};
  for (const void* f : fns) {
    const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  const void* fh[] = {QUOKA_SCORER_NB(128, kModeHeads), QUOKA_SCORER_NB(64, kModeHeads),
                      (const void*)scorer_valu_kernel<float, 128, kModeHeads>,
                      (const void*)scorer_valu_kernel<float, 64, kModeHeads>};
  for (const void* f : fh) {
    const hipError_t e =
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, bytes_heads);
    if (e != hipSuccess) return e;
  }
#undef QUOKA_SCORER_NB
  return hipSuccess;
}

// Dynamic LDS of one scorer workgroup: histogram plus the rows it reads.
size_t scorer_lds_bytes(const Problem& p) {
  const int rows = p.dtype == QUOKA_BF16 ? p.nq_pad : p.q_budget;
  return (size_t)kScoreBins * 4 + (size_t)rows * p.gh() * p.D * 4;
}

hipError_t launch_scorer(const Problem& p, const void* k_hist, char* ws, const Workspace& w,
                         float* scores, hipStream_t st) {
  if (p.NSB == 0) return hipSuccess;
  dim3 grid((unsigned)p.NSB, (unsigned)p.Hkv);
  const int32_t* plan = (const int32_t*)(ws + w.plan);
  uint32_t* hist = (uint32_t*)(ws + w.hist);
  const size_t lds = scorer_lds_bytes(p);
  const int one = p.one_row() ? 1 : 0;
  const int mode = p.mode();
  if (p.dtype == QUOKA_BF16) {
    const bf16x8* gsel = (const bf16x8*)(ws + w.gsel);
    const int nb = p.score_keys / 256;
#define QUOKA_SCORER(D, NB, M)                                                                \
  hipLaunchKernelGGL((scorer_mfma_kernel<D, NB, M>), grid, dim3(256), lds, st,                \
                     (const bf16*)k_hist, p.cu_chunk, p.cu_hist, plan, p.S, p.Hkv, p.TL,      \
                     p.q_budget, p.nq_pad, gsel, scores, hist, one, p.G)
#define QUOKA_SCORER_B(D, M)                                                                  \
  do {                                                                                        \
    if (nb == 1) QUOKA_SCORER(D, 1, M);                                                       \
    else if (nb == 2) QUOKA_SCORER(D, 2, M);                                                  \
    else if (nb == 4) QUOKA_SCORER(D, 4, M);                                                  \
    else QUOKA_SCORER(D, 8, M);                                                               \
  } while (0)
#define QUOKA_SCORER_M(D)                                                                     \
  do {                                                                                        \
    if (mode == kModeDot) QUOKA_SCORER_B(D, kModeDot);                                        \
    else if (mode == kModeHeads) QUOKA_SCORER_B(D, kModeHeads);                               \
    else QUOKA_SCORER_B(D, kModeCos);                                                         \
  } while (0)
    if (p.D == 128) QUOKA_SCORER_M(128); else QUOKA_SCORER_M(64);
#undef QUOKA_SCORER_M
#undef QUOKA_SCORER_B
#undef QUOKA_SCORER
  } else {
    const float* gsel = (const float*)(ws + w.gsel);
#define QUOKA_SCORER(D, M)                                                                    \
  hipLaunchKernelGGL((scorer_valu_kernel<float, D, M>), grid, dim3(256), lds, st,             \
                     (const float*)k_hist, p.cu_chunk, p.cu_hist, plan, p.S, p.Hkv, p.TL,     \
                     p.q_budget, p.nq_pad, gsel, scores, hist, p.score_keys, one, p.G)
#define QUOKA_SCORER_M(D)                                                                     \
  do {                                                                                        \
    if (mode == kModeDot) QUOKA_SCORER(D, kModeDot);                                          \
    else if (mode == kModeHeads) QUOKA_SCORER(D, kModeHeads);                                 \
    else QUOKA_SCORER(D, kModeCos);                                                           \
  } while (0)
    if (p.D == 128) QUOKA_SCORER_M(128); else QUOKA_SCORER_M(64);
#undef QUOKA_SCORER_M
#undef QUOKA_SCORER
  }
  return hipGetLastError();
}

}  // namespace quoka
