// Query side of QUOKA's selection: tile planning, query pre-aggregation,
// cosine to the chunk's mean query, and the N_q lowest-cosine subselection.
//
// Sources: QUOKA paper summary (hw-hk.tistory.com/367), "QUOKA Method >
// Query Subselection" (rank queries by their negative cosine to the mean
// query, keep the top N_q) and "Aggregation Across Queries and KV Groups"
// (normalised queries are averaged over the KV group before scoring);
// "QUOKA Explained", "Pick the queries that disagree with the crowd" and
// "A wrinkle: grouped-query attention".
#include "common.h"
#include "internal.h"
#include "radix.h"

namespace quoka {

// ---------------------------------------------------------------------------
// Plan: per-sequence tile prefix sums for the three tilings, and clearing of
// the counters the later kernels accumulate into. Query prep does both (its
// block (0, 0) plans, all its blocks clear a slice of [zero_begin, zero_end));
// the plan kernel covers calls where no chunk has a token.
// ---------------------------------------------------------------------------
// Tile prefix sums of the three tilings, by one thread.
__device__ void write_plan(const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist,
                           int S, int score_keys, int32_t* __restrict__ plan) {
  int32_t* qt = plan;
  int32_t* sb = plan + (S + 1);
  int32_t* kt = plan + 2 * (S + 1);
  int32_t a = 0, b = 0, c = 0;
  for (int s = 0; s < S; ++s) {
    qt[s] = a; sb[s] = b; kt[s] = c;
    const int C = cu_chunk[s + 1] - cu_chunk[s];
    const int L = cu_hist[s + 1] - cu_hist[s];
    a += (C + kQprepTokens - 1) / kQprepTokens;
    b += (L + score_keys - 1) / score_keys;
    c += (L + kTopbKeys - 1) / kTopbKeys;
  }
  qt[S] = a; sb[S] = b; kt[S] = c;
}

// Used only when no chunk has a token (so query prep, which otherwise plans
// and clears, has no workgroup).
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu_chunk,
                                                   const int32_t* __restrict__ cu_hist, int S,
                                                   int score_keys, int32_t* __restrict__ plan,
                                                   uint4* __restrict__ zero, int64_t nzero16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nzero16;
       i += (int64_t)gridDim.x * blockDim.x)
    zero[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x == 0) write_plan(cu_chunk, cu_hist, S, score_keys, plan);
}


// ---------------------------------------------------------------------------
// K1a: g_t = mean_j unit(q_{t,j}) over the G query heads of KV head h, for a
// tile of 64 tokens; also the tile's fp64 sum of g (for the mean query).
// 16 waves; each wave owns 4 tokens and issues all their row loads before
// reducing. Lanes work in groups of 16 on one head row (4 rows/instruction).
// ---------------------------------------------------------------------------
constexpr int kQprepThreads = 1024;
constexpr int kQprepWaves = kQprepThreads / 64;
constexpr int kTokPerWave = kQprepTokens / kQprepWaves;  // 4

// EPL consecutive elements as fp32, with 16-byte (or 8-byte) vector loads.
template <typename T, int EPL>
__device__ __forceinline__ void load_row(const T* __restrict__ p, float (&x)[EPL]) {
  if constexpr (sizeof(T) == 2) {
    static_assert(EPL % 4 == 0, "bf16 rows load 4 or 8 elements");
    if constexpr (EPL == 8) {
      const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
    } else {
      const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 v = *(const float4*)(p + e);
      x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kQprepThreads) void qprep_g_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ cu_chunk,
    const int32_t* __restrict__ cu_hist, int S, int Hq, int Hkv, int G, float* __restrict__ g,
    double* __restrict__ gpart, int score_keys, int32_t* __restrict__ plan,
    uint4* __restrict__ zero, int64_t nzero16) {
  constexpr int EPL = D / 16;  // elements per lane
  const int tile = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the plan and the cleared counters are for the later kernels
  {
    const int64_t nb = (int64_t)gridDim.x * gridDim.y;
    for (int64_t i = ((int64_t)h * gridDim.x + tile) * kQprepThreads + threadIdx.x; i < nzero16;
         i += nb * kQprepThreads)
      zero[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tile == 0 && h == 0 && threadIdx.x == 0) write_plan(cu_chunk, cu_hist, S, score_keys, plan);
  }
  // this tile's sequence: wave prefix sums over the sequences' tile counts
  int s = 0, t_base = 0;
  for (int s0 = 0, acc = 0; s0 < S; s0 += 64) {
    const int sq = s0 + lane;
    const int n = sq < S ? (cu_chunk[sq + 1] - cu_chunk[sq] + kQprepTokens - 1) / kQprepTokens : 0;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int excl = incl - n;
    const uint64_t m = __ballot(n > 0 && acc + excl <= tile && tile < acc + incl);
    if (m) {
      const int l = __ffsll((unsigned long long)m) - 1;
      s = s0 + l;
      t_base = acc + __shfl(excl, l, 64);
      break;
    }
    acc += __shfl(incl, 63, 64);
  }
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int grp = lane >> 4, sub = lane & 15;
  const int tw = (tile - t_base) * kQprepTokens + wave * kTokPerWave;

  float acc[kTokPerWave][EPL];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;

  for (int j0 = 0; j0 < G; j0 += 4) {
    const int j = j0 + grp;
    float x[kTokPerWave][EPL];
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
      const int t = tw + i;
      const bool ok = t < C && j < G;
      const T* row = q + ((int64_t)(c_off + (ok ? t : 0)) * Hq + (int64_t)h * G + (ok ? j : 0)) * D +
                     sub * EPL;
      load_row<T, EPL>(row, x[i]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[i][e] = ok ? x[i][e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss = fmaf(x[i][e], x[i][e], ss);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
      const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = fmaf(x[i][e], inv, acc[i][e]);
    }
  }
  double part[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[e] = 0.0;
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int t = tw + i;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[i][e];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      acc[i][e] = v / (float)G;
    }
    if (grp == 0 && t < C) {
      float* dst = g + ((int64_t)(c_off + t) * Hkv + h) * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *(float4*)(dst + e) = make_float4(acc[i][e], acc[i][e + 1], acc[i][e + 2], acc[i][e + 3]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[e] += (double)acc[i][e];
    }
  }
  __shared__ double red[kQprepWaves][D];
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[wave][sub * EPL + e] = part[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    double a = 0.0;
#pragma unroll
    for (int w = 0; w < kQprepWaves; ++w) a += red[w][threadIdx.x];
    gpart[((int64_t)tile * Hkv + h) * D + threadIdx.x] = a;
  }
}

// ---------------------------------------------------------------------------
// K2: keep the N_q,eff tokens with the lowest cosine (ties to the lower
// token) by an exact radix select over the unique keys
// (order_key(c) << 32 | t), write them ascending, and lay out the kept g rows
// for the scorer: bf16 hi/lo pairs in MFMA A-operand order, or fp32 rows.
// ---------------------------------------------------------------------------
constexpr int kQselCap = 12288;  // chunk tokens whose cosines are staged in LDS

template <int D, bool kMfma>
__device__ void select_kept_queries(int prob, int h, int Hkv, int c_off, int C, int q_budget,
                                    int nq_pad, const float* __restrict__ src_g,
                                    const float* __restrict__ g, int32_t* __restrict__ qidx,
                                    void* __restrict__ gsel, float* cs,
                                    RadixScratch<kQprepThreads>& rs, int32_t* kept) {
  constexpr int NT = kQprepThreads;
  const int n = min(q_budget, C);
  int32_t* out = qidx + (int64_t)prob * q_budget;
  const float* src = src_g;
  if (C <= kQselCap) {
    block_copy<NT, 4>(cs, src, C);
    src = cs;
  }
  __syncthreads();
  auto key_of = [&](int t) -> uint64_t {
    return ((uint64_t)float_order_key(src[t]) << 32) | (uint32_t)t;
  };
  uint64_t prefix = ~0ull, mask = ~0ull;  // keep everything when n == C
  if (n < C) radix_select<false, NT>(key_of, C, n, rs, prefix, mask);

  // ascending compaction of the kept tokens
  const int per = (C + NT - 1) / NT;
  const int b0 = threadIdx.x * per, b1 = min(C, b0 + per);
  uint32_t cnt = 0;
  for (int t = b0; t < b1; ++t) cnt += radix_taken<false>(key_of(t), prefix, mask);
  uint32_t pos = block_exclusive_scan<NT>(cnt, rs);
  for (int t = b0; t < b1; ++t) {
    if (radix_taken<false>(key_of(t), prefix, mask)) {
      out[pos] = t;
      kept[pos] = t;
      ++pos;
    }
  }
  for (int i = n + threadIdx.x; i < q_budget; i += NT) out[i] = -1;
  if (n == 0) return;  // empty chunk: the scorer writes zero scores
  __syncthreads();

  if constexpr (kMfma) {
    // A operand of v_mfma_f32_16x16x32_bf16: lane l holds row l%16 and the
    // 8 d-values (l/16)*8.. of the 32-wide d-step; layout
    // [qb][ds][term: hi, lo][lane] of bf16x8. Rows past n repeat row 0,
    // which leaves the max over kept tokens unchanged.
    constexpr int NDS = D / 32;
    bf16x8* dst = (bf16x8*)gsel + (int64_t)prob * (nq_pad / 16) * NDS * 2 * 64;
    const int total = (nq_pad / 16) * NDS * 64;
    for (int v = threadIdx.x; v < total; v += NT) {
      const int lane = v & 63, rest = v >> 6;  // rest = qb * NDS + ds
      const int row = (rest / NDS) * 16 + (lane & 15);
      const int d0 = (rest % NDS) * 32 + (lane >> 4) * 8;
      const int t = kept[row < n ? row : 0];
      const float4* gp = (const float4*)(g + ((int64_t)(c_off + t) * Hkv + h) * D + d0);
      const float4 x0 = gp[0], x1 = gp[1];
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = (bf16)x[e];
        lo[e] = (bf16)(x[e] - (float)hi[e]);
      }
      dst[(rest * 2 + 0) * 64 + lane] = hi;
      dst[(rest * 2 + 1) * 64 + lane] = lo;
    }
  } else {
    float* dst = (float*)gsel + (int64_t)prob * nq_pad * D;
    for (int idx = threadIdx.x; idx < n * D; idx += NT) {
      const int row = idx / D, d = idx % D;
      dst[idx] = g[((int64_t)(c_off + kept[row]) * Hkv + h) * D + d];
    }
  }
}

// ---------------------------------------------------------------------------
// K1b: c_t = cos(M, g_t) for a tile of 64 tokens, fp64 dot products. Every
// workgroup forms M = (1/C) sum_t g_t itself from the tile sums, in a fixed
// order (a device-scope hand-off from one workgroup to the others would cost
// an L2 write-back per workgroup on this chip, more than the repeated sum).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kQprepThreads) void qprep_cos_kernel(
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TC, const float* __restrict__ g, const double* __restrict__ gpart,
    float* __restrict__ qcos) {
  constexpr int P = kQprepThreads / D;  // partial sums per channel
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* qt_off = plan;
  const int s = upper_seq(qt_off, S, tile);
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ double parts[P][D];
  __shared__ double Md[D];
  __shared__ double red[kQprepWaves];
  {
    const int d = threadIdx.x % D, pp = threadIdx.x / D;
    const int k0 = qt_off[s], k1 = qt_off[s + 1];
    double a = 0.0;
    for (int k = k0 + pp; k < k1; k += 4 * P) {
      double v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kk = k + u * P;
        v[u] = kk < k1 ? gpart[((int64_t)kk * Hkv + h) * D + d] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) a += v[u];
    }
    parts[pp][d] = a;
  }
  __syncthreads();
  double sq = 0.0;
  if (threadIdx.x < D) {
    double a = 0.0;
#pragma unroll
    for (int pp = 0; pp < P; ++pp) a += parts[pp][threadIdx.x];
    a /= (double)C;
    Md[threadIdx.x] = a;
    sq = a * a;
  }
  sq = wave_sum(sq);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  double msq = 0.0;
#pragma unroll
  for (int w = 0; w < kQprepWaves; ++w) msq += red[w];
  const double mnorm = sqrt(msq);

  constexpr int EPL = D / 64;
  double m[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) m[e] = Md[lane * EPL + e];
  const int tw = (tile - qt_off[s]) * kQprepTokens + wave * kTokPerWave;
  float x[kTokPerWave][EPL];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int t = tw + i;
    const float* gr = g + ((int64_t)(c_off + (t < C ? t : 0)) * Hkv + h) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[i][e] = gr[e];
  }
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    double dot = 0.0, gg = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const double v = (double)x[i][e];
      dot += v * m[e];
      gg += v * v;
    }
    dot = wave_sum(dot);
    gg = wave_sum(gg);
    const int t = tw + i;
    if (lane == 0 && t < C) {
      const double den = mnorm * sqrt(gg);
      qcos[(int64_t)h * TC + c_off + t] = den > 0.0 ? (float)(dot / den) : 0.f;
    }
  }
}

// One workgroup per (sequence, KV head): the query select, plus the -1
// padding of sel_idx past B_eff (the top-B select writes [0, B_eff)).
template <int D, bool kMfma>
__global__ __launch_bounds__(kQprepThreads) void qselect_kernel(
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist, int Hkv, int64_t TC,
    const float* __restrict__ g, const float* __restrict__ qcos, int q_budget, int nq_pad,
    int32_t* __restrict__ qidx, void* __restrict__ gsel, int kv_budget,
    int32_t* __restrict__ sel_idx) {
  const int prob = blockIdx.x, s = prob / Hkv, h = prob % Hkv;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  {
    const int L = cu_hist[s + 1] - cu_hist[s];
    int32_t* srow = sel_idx + (int64_t)prob * kv_budget;
    for (int i = min(kv_budget, L) + threadIdx.x; i < kv_budget; i += kQprepThreads) srow[i] = -1;
  }
  __shared__ float cs[kQselCap];
  __shared__ int32_t kept[QUOKA_MAX_Q_BUDGET];
  __shared__ RadixScratch<kQprepThreads> rs;
  select_kept_queries<D, kMfma>(prob, h, Hkv, c_off, C, q_budget, nq_pad,
                                qcos + (int64_t)h * TC + c_off, g, qidx, gsel, cs, rs, kept);
}

hipError_t launch_qprep(const Problem& p, const void* q, char* ws, const Workspace& w,
                        float* qcos, int32_t* qidx, int32_t* sel_idx, hipStream_t st) {
  int32_t* plan = (int32_t*)(ws + w.plan);
  float* g = (float*)(ws + w.g);
  double* gpart = (double*)(ws + w.gpart);
  uint4* zero = (uint4*)(ws + w.zero_begin);
  const int64_t n16 = (int64_t)((w.zero_end - w.zero_begin) / 16);
  const dim3 block(kQprepThreads);
  if (p.NQT == 0) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, p.cu_chunk, p.cu_hist, p.S,
                       p.score_keys, plan, zero, n16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    dim3 grid((unsigned)p.NQT, (unsigned)p.Hkv);
#define QUOKA_QPREP(T, D)                                                                     \
  hipLaunchKernelGGL((qprep_g_kernel<T, D>), grid, block, 0, st, (const T*)q, p.cu_chunk,     \
                     p.cu_hist, p.S, p.Hq, p.Hkv, p.G, g, gpart, p.score_keys, plan, zero, n16)
    if (p.dtype == QUOKA_BF16) {
      if (p.D == 128) QUOKA_QPREP(bf16, 128); else QUOKA_QPREP(bf16, 64);
    } else {
      if (p.D == 128) QUOKA_QPREP(float, 128); else QUOKA_QPREP(float, 64);
    }
#undef QUOKA_QPREP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.D == 128)
      hipLaunchKernelGGL((qprep_cos_kernel<128>), grid, block, 0, st, p.cu_chunk, plan, p.S,
                         p.Hkv, p.TC, g, gpart, qcos);
    else
      hipLaunchKernelGGL((qprep_cos_kernel<64>), grid, block, 0, st, p.cu_chunk, plan, p.S,
                         p.Hkv, p.TC, g, gpart, qcos);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 sgrid((unsigned)(p.S * p.Hkv));
#define QUOKA_QSEL(D, M)                                                                      \
  hipLaunchKernelGGL((qselect_kernel<D, M>), sgrid, block, 0, st, p.cu_chunk, p.cu_hist, p.Hkv, \
                     p.TC, g, qcos, p.q_budget, p.nq_pad, qidx, (void*)(ws + w.gsel),         \
                     p.kv_budget, sel_idx)
  const bool mfma = p.dtype == QUOKA_BF16;
  if (p.D == 128) { if (mfma) QUOKA_QSEL(128, true); else QUOKA_QSEL(128, false); }
  else            { if (mfma) QUOKA_QSEL(64, true);  else QUOKA_QSEL(64, false); }
#undef QUOKA_QSEL
  return hipGetLastError();
}

}  // namespace quoka
