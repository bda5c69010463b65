// Query side of QUOKA's selection: tile planning, query pre-aggregation,
// cosine to the chunk's mean query, and the N_q lowest-cosine subselection.
//
// Sources: QUOKA paper summary (hw-hk.tistory.com/367), "QUOKA Method >
// Query Subselection" (rank queries by their negative cosine to the mean
// query, keep the top N_q) and "Aggregation Across Queries and KV Groups"
// (normalised queries are averaged over the KV group before scoring);
// "QUOKA Explained", "Pick the queries that disagree with the crowd" and
// "A wrinkle: grouped-query attention".
#include <type_traits>

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
                           int S, int qtok, int score_keys, int32_t* __restrict__ plan) {
  int32_t* qt = plan;
  int32_t* sb = plan + (S + 1);
  int32_t* kt = plan + 2 * (S + 1);
  int32_t a = 0, b = 0, c = 0;
  for (int s = 0; s < S; ++s) {
    qt[s] = a; sb[s] = b; kt[s] = c;
    const int C = cu_chunk[s + 1] - cu_chunk[s];
    const int L = cu_hist[s + 1] - cu_hist[s];
    a += (C + qtok - 1) / qtok;
    b += (L + score_keys - 1) / score_keys;
    c += (L + kTopbKeys - 1) / kTopbKeys;
  }
  qt[S] = a; sb[S] = b; kt[S] = c;
}

// Used only when no chunk has a token (so query prep, which otherwise plans
// and clears, has no workgroup).
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu_chunk,
                                                   const int32_t* __restrict__ cu_hist, int S,
                                                   int qtok, int score_keys, int32_t* __restrict__ plan,
                                                   uint4* __restrict__ zero, int64_t nzero16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nzero16;
       i += (int64_t)gridDim.x * blockDim.x)
    zero[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x == 0) write_plan(cu_chunk, cu_hist, S, qtok, score_keys, plan);
}


// ---------------------------------------------------------------------------
// K1a: g_t = mean_j unit(q_{t,j}) over the G query heads of KV head h, for a
// tile of 16 kTokPerWave tokens (64, or 32 / 16 for shapes with few tiles);
// also the tile's fp64 sum of g (for the mean query). 16 waves; each wave
// owns kTokPerWave tokens and issues all their row loads before reducing. A head row is spread over D / 4 lanes (4 elements each), so one
// load instruction covers 256 / D rows; the arithmetic is fp64.
// ---------------------------------------------------------------------------
constexpr int kQprepThreads = kQprepWavesTotal * 64;
constexpr int kQprepWaves = kQprepWavesTotal;

// 4 consecutive elements as fp32 (one 8- or 16-byte load).
template <typename T>
__device__ __forceinline__ void load4(const T* __restrict__ p, float (&x)[4]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
  } else {
    const float4 v = *(const float4*)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
}

// 1/sqrt(x) in fp64 for x > 0: the hardware estimate refined by two
// Newton-Raphson steps r <- r (3 - x r^2) / 2, each of which squares the
// estimate's relative error, so the result is the fp64 value to a few units
// in the last place (about half the cost of a correctly rounded sqrt and a
// division).
__device__ __forceinline__ double rsqrt_f64(double x) {
  double r = __builtin_amdgcn_rsq(x);
  const double hx = -0.5 * x;
  r = r * fma(hx, r * r, 1.5);
  r = r * fma(hx, r * r, 1.5);
  return r;
}

// Sum over the RL lanes of one head row (aligned groups of RL = 16 or 32).
template <int RL>
__device__ __forceinline__ double head_row_sum(double v) {
  v = row16_sum(v);
  return RL == 32 ? pair16_sum(v) : v;
}
// Sum over the 64 / RL head rows of one load instruction (lanes l, l + RL, ...).
template <int RL>
__device__ __forceinline__ double head_group_sum(double v) {
  return RL == 32 ? pair32_sum(v) : rows_sum(v);
}

template <typename T, int D, int kTokPerWave>
__global__ __launch_bounds__(kQprepThreads) void qprep_g_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ cu_chunk,
    const int32_t* __restrict__ cu_hist, int S, int Hq, int Hkv, int G, float* __restrict__ g,
    double* __restrict__ gpart, int score_keys, int32_t* __restrict__ plan,
    uint4* __restrict__ zero, int64_t nzero16) {
  constexpr int EPL = 4;       // elements per lane
  constexpr int RL = D / EPL;  // lanes per head row: 32 or 16
  constexpr int RPI = 64 / RL; // head rows per load instruction
  constexpr int kQprepTok = kQprepWaves * kTokPerWave;  // tokens per tile
  const int tile = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the plan and the cleared counters are for the later kernels
  {
    const int64_t nb = (int64_t)gridDim.x * gridDim.y;
    for (int64_t i = ((int64_t)h * gridDim.x + tile) * kQprepThreads + threadIdx.x; i < nzero16;
         i += nb * kQprepThreads)
      zero[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tile == 0 && h == 0 && threadIdx.x == 0)
      write_plan(cu_chunk, cu_hist, S, kQprepTok, score_keys, plan);
  }
  // this tile's sequence: wave prefix sums over the sequences' tile counts
  int s = 0, t_base = 0;
  for (int s0 = 0, acc = 0; s0 < S; s0 += 64) {
    const int sq = s0 + lane;
    const int n = sq < S ? (cu_chunk[sq + 1] - cu_chunk[sq] + kQprepTok - 1) / kQprepTok : 0;
    const int incl = (int)wave_inclusive_scan((uint32_t)n);
    const int excl = incl - n;
    const uint64_t m = __ballot(n > 0 && acc + excl <= tile && tile < acc + incl);
    if (m) {
      const int l = __ffsll((unsigned long long)m) - 1;
      s = s0 + l;
      t_base = acc + __builtin_amdgcn_readlane(excl, l);
      break;
    }
    acc += __builtin_amdgcn_readlane(incl, 63);
  }
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int grp = lane / RL, sub = lane % RL;
  const int tw = (tile - t_base) * kQprepTok + wave * kTokPerWave;

  // the unit head rows and their mean over the group in fp64, so that the
  // tile sums (hence the mean query) and the stored g (rounded once to fp32)
  // are the fp64 values up to rounding
  double acc[kTokPerWave][EPL];
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = 0.0;

  for (int j0 = 0; j0 < G; j0 += RPI) {
    const int j = j0 + grp;
    float x[kTokPerWave][EPL];
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
      const int t = tw + i;
      const bool ok = t < C && j < G;
      const T* row = q + ((int64_t)(c_off + (ok ? t : 0)) * Hq + (int64_t)h * G + (ok ? j : 0)) * D +
                     sub * EPL;
      load4<T>(row, x[i]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) x[i][e] = ok ? x[i][e] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
      double ss = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss = fma((double)x[i][e], (double)x[i][e], ss);
      ss = head_row_sum<RL>(ss);
      const double inv = ss > 0.0 ? rsqrt_f64(ss) : 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = fma((double)x[i][e], inv, acc[i][e]);
    }
  }
  double part[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[e] = 0.0;
#pragma unroll
  for (int i = 0; i < kTokPerWave; ++i) {
    const int t = tw + i;
    // the mean over the group: for a power-of-two G the product with 1/G is
    // the same correctly rounded value as the quotient, at one instruction
    if ((G & (G - 1)) == 0) {
      const double inv_g = 1.0 / (double)G;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = head_group_sum<RL>(acc[i][e]) * inv_g;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[i][e] = head_group_sum<RL>(acc[i][e]) / (double)G;
    }
    if (grp == 0 && t < C) {
      float* dst = g + ((int64_t)(c_off + t) * Hkv + h) * D + sub * EPL;
      *(float4*)dst = make_float4((float)acc[i][0], (float)acc[i][1], (float)acc[i][2],
                                  (float)acc[i][3]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[e] += acc[i][e];
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
// token), as the fp64 cosines order them, and write them ascending to out
// and kept. Returns N_q,eff.
//
// src holds fp32 cosines within err of the fp64 values. An exact radix select
// over the unique keys (order_key(c) << 32 | t) decides every token except
// those within 2 err of the N_q,eff-th value: if that band holds more tokens
// than the places left for it, their cosines are recomputed in fp64
// (exact_cos, one wave per token) and the selection is redone over class
// keys (tokens surely in, then the band by fp64 value, then the rest) kept
// in kbuf [C].
// ---------------------------------------------------------------------------
// Exclusive prefix sum of cnt over the block, and the block's maximum of mx
// and minimum of mn, in one exchange through LDS.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_max_min(uint32_t cnt, uint32_t& mx, uint32_t& mn,
                                                       RadixScratch<NT>& rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(cnt);
  const uint32_t wmx = ~wave_min(~mx), wmn = wave_min(mn);
  if (lane == 63) rs.wsum[w] = x;
  if (lane == 0) {
    rs.wand[w] = wmx;
    rs.wor[w] = wmn;
  }
  __syncthreads();
  uint32_t add = 0, bmx = 0u, bmn = ~0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    if (i < w) add += rs.wsum[i];
    bmx = max(bmx, (uint32_t)rs.wand[i]);
    bmn = min(bmn, (uint32_t)rs.wor[i]);
  }
  __syncthreads();
  mx = bmx;
  mn = bmn;
  return x - cnt + add;
}

template <int NT, typename ExactFn>
__device__ int select_tokens(int C, int q_budget, const float* __restrict__ src, float* cs,
                             RadixScratch<NT>& rs, float err, uint64_t* __restrict__ kbuf,
                             ExactFn exact_cos, int32_t* __restrict__ out, int32_t* kept) {
  const int n = min(q_budget, C);
  if (C <= kQselCap && src != cs) {
    block_copy<NT, 8>(cs, src, C);  // up to 8 NT cosines in one round of loads
    src = cs;
  }
  __syncthreads();
  auto approx_key = [&](int t) -> uint64_t {
    return ((uint64_t)float_order_key(src[t]) << 32) | (uint32_t)t;
  };
  uint64_t prefix = ~0ull, mask = ~0ull;  // keep everything when n == C
  bool use_k = false;
  if (n < C) radix_select<false, NT>(approx_key, C, n, rs, prefix, mask);
  auto key_of = [&](int t) -> uint64_t { return use_k ? kbuf[t] : approx_key(t); };

  // ascending compaction of the kept tokens (each thread a contiguous range);
  // the same pass finds cn, the n-th lowest fp32 cosine, and the lowest one
  // left out
  const int per = (C + NT - 1) / NT;
  const int b0 = threadIdx.x * per, b1 = min(C, b0 + per);
  uint32_t cnt = 0, kn = 0u, kout = ~0u;
  for (int t = b0; t < b1; ++t) {
    const uint64_t k = approx_key(t);
    if (radix_taken<false>(k, prefix, mask)) {
      ++cnt;
      kn = max(kn, (uint32_t)(k >> 32));
    } else {
      kout = min(kout, (uint32_t)(k >> 32));
    }
  }
  uint32_t pos = block_scan_max_min<NT>(cnt, kn, kout, rs);
  if (n < C) {
    // when every token left out lies more than 2 err above cn, the fp32
    // selection is the fp64 one; else the band within 2 err of cn is re-ranked
    const double cn = (double)float_from_order_key(kn);
    const double lo = cn - 2.0 * (double)err, hi = cn + 2.0 * (double)err;
    if ((double)float_from_order_key(kout) <= hi) {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      for (int t0 = wave * 64; t0 < C; t0 += NT) {
        const int t = t0 + lane;
        const double c = t < C ? (double)src[t] : 0.0;
        const bool band = t < C && c >= lo && c <= hi;
        if (t < C && !band) kbuf[t] = class_key_asc(c < lo ? 0u : 2u, 0.0, t);
        uint64_t m = __ballot(band);
        while (m) {
          const int l = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const double ce = exact_cos(t0 + l);
          if (lane == 0) kbuf[t0 + l] = class_key_asc(1u, ce, t0 + l);
        }
      }
      __syncthreads();
      radix_select<false, NT>([&](int t) { return kbuf[t]; }, C, n, rs, prefix, mask);
      use_k = true;
      cnt = 0;
      for (int t = b0; t < b1; ++t) cnt += radix_taken<false>(key_of(t), prefix, mask);
      pos = block_exclusive_scan<NT>(cnt, rs);
    }
  }
  for (int t = b0; t < b1; ++t) {
    if (radix_taken<false>(key_of(t), prefix, mask)) {
      out[pos] = t;
      kept[pos] = t;
      ++pos;
    }
  }
  for (int i = n + threadIdx.x; i < q_budget; i += NT) out[i] = -1;
  return n;
}

// The fp64 cosine of token row `tok` (c_off + t) of KV head h to the chunk's
// mean query, by one wave (the value in every lane): g = mean_j unit(q_j)
// over the group's heads, M = (1/C) sum of the fp64 tile sums of g (tiles
// [k0, k1) of the chunk).
template <typename T, int D>
__device__ double exact_token_cos(const T* __restrict__ q, int64_t tok, int Hq, int h, int G,
                                  const double* __restrict__ gpart, int Hkv, int k0, int k1,
                                  int C) {
  constexpr int EPL = D / 64;
  const int lane = threadIdx.x & 63;
  double m[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) m[e] = 0.0;
  for (int k = k0; k < k1; ++k)
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] += gpart[((int64_t)k * Hkv + h) * D + lane * EPL + e];
  double g[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    m[e] /= (double)C;
    g[e] = 0.0;
  }
  for (int j = 0; j < G; ++j) {
    const T* row = q + (tok * Hq + (int64_t)h * G + j) * D + lane * EPL;
    double x[EPL], ss = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      x[e] = (double)to_f32(row[e]);
      ss = fma(x[e], x[e], ss);
    }
    ss = wave_sum(ss);
    const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) g[e] = fma(x[e], inv, g[e]);
  }
  double dot = 0.0, gg = 0.0, mm = 0.0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    g[e] /= (double)G;
    dot = fma(g[e], m[e], dot);
    gg = fma(g[e], g[e], gg);
    mm = fma(m[e], m[e], mm);
  }
  dot = wave_sum(dot);
  gg = wave_sum(gg);
  mm = wave_sum(mm);
  const double den = sqrt(mm) * sqrt(gg);
  return den > 0.0 ? dot / den : 0.0;
}

// 8 consecutive elements of a row as fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* __restrict__ p, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else {
    const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// ---------------------------------------------------------------------------
// K1b: c_t = cos(M, g_t) for a query-prep tile, fp64 dot products. Every
// workgroup forms M = (1/C) sum_t g_t itself from the tile sums, in a fixed
// order (a device-scope hand-off from one workgroup to the others would cost
// an L2 write-back per workgroup on this chip, more than the repeated sum).
// ---------------------------------------------------------------------------
template <int D, int kTokPerWave>
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
  const double minv = msq > 0.0 ? rsqrt_f64(msq) : 0.0;  // 1 / |M|

  constexpr int EPL = D / 64;
  double m[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) m[e] = Md[lane * EPL + e];
  const int tw = (tile - qt_off[s]) * (kQprepWaves * kTokPerWave) + wave * kTokPerWave;
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
      const double ginv = gg > 0.0 ? rsqrt_f64(gg) : 0.0;  // 1 / |g_t|
      qcos[(int64_t)h * TC + c_off + t] = (float)(dot * ginv * minv);
    }
  }
}

// One workgroup per (sequence, KV head): the query select, the -1 padding of
// sel_idx past B_eff (the top-B select writes [0, B_eff)), and the rows the
// scorer reads, laid out per variant:
//   QUOKA, GLOBAL      g_t of the kept tokens
//   DOT                (1/G) sum_j q_{t,j} of the kept tokens
//   PER_HEAD           unit(q_{t,j}) for every head j of the kept tokens
//   MEAN_QUERIES       one row, the mean of the kept tokens' g_t
//   MEAN_QUERY         one row, the chunk's mean query M (no subselection)
// bf16 (kMfma): hi/lo bf16 pairs in MFMA A-operand order, 16-row blocks,
// layout [block][head][d-step][term][lane] of bf16x8; rows past the last
// repeat row 0 (which leaves a max unchanged). fp32: rows [row][head][d].
constexpr int kQselThreads = 512;  // threads of the one workgroup per (sequence, KV head)

template <int D, bool kMfma>
__global__ __launch_bounds__(kQselThreads) void qselect_kernel(
    const void* __restrict__ qv, const int32_t* __restrict__ cu_chunk,
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int Hq, int Hkv,
    int G, int64_t TC, const float* __restrict__ g, const double* __restrict__ gpart,
    const float* __restrict__ qcos, int q_budget, int nq_pad, int variant,
    int32_t* __restrict__ qidx, void* __restrict__ gsel, int kv_budget,
    int32_t* __restrict__ sel_idx, float cos_err, uint64_t* __restrict__ qkey,
    double* __restrict__ row0) {
  using T = typename std::conditional<kMfma, bf16, float>::type;
  constexpr int NT = kQselThreads;
  const T* q = (const T*)qv;
  const int prob = blockIdx.x, s = prob / Hkv, h = prob % Hkv;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  {
    const int L = cu_hist[s + 1] - cu_hist[s];
    int32_t* srow = sel_idx + (int64_t)prob * kv_budget;
    for (int i = min(kv_budget, L) + threadIdx.x; i < kv_budget; i += NT) srow[i] = -1;
  }
  __shared__ float cs[kQselCap];
  __shared__ int32_t kept[QUOKA_MAX_Q_BUDGET];
  __shared__ RadixScratch<NT> rs;
  __shared__ float mrow[D];
  __shared__ double wpart[kQselThreads / 64][D];
  __shared__ float inv_norm[kMaxHeadRows];
  int32_t* out = qidx + (int64_t)prob * q_budget;
  const bool one = variant == QUOKA_VARIANT_MEAN_QUERIES || variant == QUOKA_VARIANT_MEAN_QUERY;
  const int GH = variant == QUOKA_VARIANT_PER_HEAD ? G : 1;

  int n;
  if (variant == QUOKA_VARIANT_MEAN_QUERY) {
    for (int i = threadIdx.x; i < q_budget; i += NT) out[i] = -1;
    if (C == 0) return;  // the scorer writes zero scores
    n = 1;
    if (threadIdx.x < D) {  // M = (1/C) sum of the tile sums, in tile order
      const int32_t* qt_off = plan;
      double a = 0.0;
      for (int k = qt_off[s]; k < qt_off[s + 1]; ++k)
        a += gpart[((int64_t)k * Hkv + h) * D + threadIdx.x];
      a /= (double)C;
      mrow[threadIdx.x] = (float)a;
      row0[(int64_t)prob * D + threadIdx.x] = a;
    }
  } else {
    const float* src = qcos + (int64_t)h * TC + c_off;
    const bool global = variant == QUOKA_VARIANT_GLOBAL;
    // the fp32 cosines are within cos_err of the fp64 ones; the head average
    // of the cross-head baseline adds its own fp32 sums and quotient
    float err = cos_err;
    if (global) {  // C <= kQselCap (checked on the host)
      for (int t = threadIdx.x; t < C; t += NT) {
        float a = 0.f;
        for (int hh = 0; hh < Hkv; ++hh) a += qcos[(int64_t)hh * TC + c_off + t];
        cs[t] = a / (float)Hkv;
      }
      src = cs;
      err += (float)(Hkv + 2) * 0x1p-24f;
    }
    const int k0 = plan[s], k1 = plan[s + 1];  // this chunk's query-prep tiles
    auto exact_cos = [&](int t) -> double {
      if (!global) return exact_token_cos<T, D>(q, c_off + t, Hq, h, G, gpart, Hkv, k0, k1, C);
      double a = 0.0;
      for (int hh = 0; hh < Hkv; ++hh)
        a += exact_token_cos<T, D>(q, c_off + t, Hq, hh, G, gpart, Hkv, k0, k1, C);
      return a / (double)Hkv;
    };
    n = select_tokens<NT>(C, q_budget, src, cs, rs, err, qkey + (int64_t)h * TC + c_off,
                          exact_cos, out, kept);
    if (n == 0) return;  // empty chunk: the scorer writes zero scores
    __syncthreads();
    if (variant == QUOKA_VARIANT_MEAN_QUERIES) {
      // the mean over the kept tokens of g_t in fp64, from the query rows:
      // quad u (four lanes, D / 4 dims each) takes tokens u, u + 128, ...
      constexpr int QE = D / 4, QL = QE / 8;
      const int quad = threadIdx.x >> 2, ql = threadIdx.x & 3;
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
      double gs[QE];
#pragma unroll
      for (int e = 0; e < QE; ++e) gs[e] = 0.0;
      for (int r = quad; r < n; r += NT / 4) {
        const T* qt = q + ((int64_t)(c_off + kept[r]) * Hq + (int64_t)h * G) * D + ql * QE;
        for (int j = 0; j < G; ++j) {
          Raw8<T> x[QL];
#pragma unroll
          for (int u = 0; u < QL; ++u) x[u].load(qt + (int64_t)j * D + u * 8);
          double xx = 0.0;
#pragma unroll
          for (int u = 0; u < QL; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) xx = fma(x[u][e], x[u][e], xx);
          xx = quad_sum(xx);
          const double inv = xx > 0.0 ? 1.0 / sqrt(xx) : 0.0;
#pragma unroll
          for (int u = 0; u < QL; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) gs[u * 8 + e] = fma(x[u][e], inv, gs[u * 8 + e]);
        }
      }
      // the wave's 16 quads (row_ror 4 and 8 inside each row, then the four
      // rows), then the waves through LDS
#pragma unroll
      for (int e = 0; e < QE; ++e) {
        double v = gs[e];
        v += dpp_f64<0x124>(v);
        v += dpp_f64<0x128>(v);
        v = rows_sum(v);
        if (lane < 4) wpart[wave][ql * QE + e] = v;
      }
      __syncthreads();
      if (threadIdx.x < D) {
        double a = 0.0;
        for (int w2 = 0; w2 < NT / 64; ++w2) a += wpart[w2][threadIdx.x];
        a /= (double)n * (double)G;
        mrow[threadIdx.x] = (float)a;
        row0[(int64_t)prob * D + threadIdx.x] = a;
      }
    } else if (variant == QUOKA_VARIANT_PER_HEAD) {  // n * G <= kMaxHeadRows (host check)
      for (int i = threadIdx.x; i < n * G; i += NT) {
        const int r = i / G, j = i % G;
        const T* row = q + ((int64_t)(c_off + kept[r]) * Hq + (int64_t)h * G + j) * D;
        float ss = 0.f;
        for (int d0 = 0; d0 < D; d0 += 8) {
          float x[8];
          load8<T>(row + d0, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        }
        inv_norm[i] = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
      }
    }
  }
  __syncthreads();

  const int nrows = one ? 1 : n;
  // 8 values (dims d0..d0+7) of row r, head j
  auto row8 = [&](int r, int j, int d0, float (&x)[8]) {
    if (one) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = mrow[d0 + e];
      return;
    }
    const int t = c_off + kept[r];
    if (variant == QUOKA_VARIANT_DOT) {
      const T* row = q + ((int64_t)t * Hq + (int64_t)h * G) * D + d0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
      for (int jj = 0; jj < G; ++jj) {
        float y[8];
        load8<T>(row + (int64_t)jj * D, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += y[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] /= (float)G;
    } else if (variant == QUOKA_VARIANT_PER_HEAD) {
      load8<T>(q + ((int64_t)t * Hq + (int64_t)h * G + j) * D + d0, x);
      const float inv = inv_norm[r * G + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= inv;
    } else {
      const float4* gp = (const float4*)(g + ((int64_t)t * Hkv + h) * D + d0);
      const float4 a = gp[0], b = gp[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
  };

  if constexpr (kMfma) {
    // A operand of v_mfma_f32_16x16x32_bf16: lane l holds row l%16 and the
    // 8 d-values (l/16)*8.. of the 32-wide d-step.
    constexpr int NDS = D / 32;
    bf16x8* dst = (bf16x8*)gsel + (int64_t)prob * (nq_pad / 16) * GH * NDS * 2 * 64;
    const int total = (nrows + 15) / 16 * GH * NDS * 64;
    // U items per thread per round, every row read issued before the first
    // conversion, so the reads of one round overlap
    constexpr int U = 4;
    for (int v0 = threadIdx.x; v0 < total; v0 += U * NT) {
      float x[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * NT;
        if (v < total) {
          const int lane = v & 63, rest = v >> 6;  // rest = (qb * GH + j) * NDS + ds
          const int ds = rest % NDS, j = (rest / NDS) % GH, qb = rest / NDS / GH;
          const int row = qb * 16 + (lane & 15);
          row8(row < nrows ? row : 0, j, ds * 32 + (lane >> 4) * 8, x[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * NT;
        if (v < total) {
          const int lane = v & 63, rest = v >> 6;
          bf16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            hi[e] = (bf16)x[u][e];
            lo[e] = (bf16)(x[u][e] - (float)hi[e]);
          }
          dst[(rest * 2 + 0) * 64 + lane] = hi;
          dst[(rest * 2 + 1) * 64 + lane] = lo;
        }
      }
    }
  } else {
    float* dst = (float*)gsel + (int64_t)prob * nq_pad * GH * D;
    const int total = nrows * GH * (D / 8);
    for (int v = threadIdx.x; v < total; v += NT) {
      const int d0 = (v % (D / 8)) * 8, rj = v / (D / 8);
      float x[8];
      row8(rj / GH, rj % GH, d0, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[(int64_t)rj * D + d0 + e] = x[e];
    }
  }
}

hipError_t launch_qprep(const Problem& p, const void* q, char* ws, const Workspace& w,
                        float* qcos, bool want_cos, int32_t* qidx, int32_t* sel_idx,
                        hipStream_t st) {
  int32_t* plan = (int32_t*)(ws + w.plan);
  float* g = (float*)(ws + w.g);
  double* gpart = (double*)(ws + w.gpart);
  uint4* zero = (uint4*)(ws + w.zero_begin);
  const int64_t n16 = (int64_t)((w.zero_end - w.zero_begin) / 16);
  const dim3 block(kQprepThreads);
  if (p.NQT == 0) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, p.cu_chunk, p.cu_hist, p.S,
                       p.qtok, p.score_keys, plan, zero, n16);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    dim3 grid((unsigned)p.NQT, (unsigned)p.Hkv);
    const int tpw = p.qtok / kQprepWaves;  // tokens per wave: 4, 2 or 1
#define QUOKA_QPREP1(T, D, TPW)                                                               \
  hipLaunchKernelGGL((qprep_g_kernel<T, D, TPW>), grid, block, 0, st, (const T*)q, p.cu_chunk, \
                     p.cu_hist, p.S, p.Hq, p.Hkv, p.G, g, gpart, p.score_keys, plan, zero, n16)
#define QUOKA_QPREP(T, D)                                                                     \
  { if (tpw == 4) QUOKA_QPREP1(T, D, 4); else if (tpw == 2) QUOKA_QPREP1(T, D, 2);            \
    else QUOKA_QPREP1(T, D, 1); }
    if (p.dtype == QUOKA_BF16) {
      if (p.D == 128) QUOKA_QPREP(bf16, 128) else QUOKA_QPREP(bf16, 64)
    } else {
      if (p.D == 128) QUOKA_QPREP(float, 128) else QUOKA_QPREP(float, 64)
    }
#undef QUOKA_QPREP
#undef QUOKA_QPREP1
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the select keeps every token of a chunk that has at most q_budget of them,
    // whatever their cosines; the mean-query baseline does not subselect at all
    const bool need_cos =
        p.variant != QUOKA_VARIANT_MEAN_QUERY && (want_cos || p.maxC > p.q_budget);
#define QUOKA_QCOS(D, TPW)                                                                    \
  hipLaunchKernelGGL((qprep_cos_kernel<D, TPW>), grid, block, 0, st, p.cu_chunk, plan, p.S,   \
                     p.Hkv, p.TC, g, gpart, qcos)
#define QUOKA_QCOS_D(D)                                                                       \
  { if (tpw == 4) QUOKA_QCOS(D, 4); else if (tpw == 2) QUOKA_QCOS(D, 2); else QUOKA_QCOS(D, 1); }
    if (need_cos) {
      if (p.D == 128) QUOKA_QCOS_D(128) else QUOKA_QCOS_D(64)
    }
#undef QUOKA_QCOS_D
#undef QUOKA_QCOS
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 sgrid((unsigned)(p.S * p.Hkv));
#define QUOKA_QSEL(D, M)                                                                      \
  hipLaunchKernelGGL((qselect_kernel<D, M>), sgrid, dim3(kQselThreads), 0, st, q, p.cu_chunk,   \
                     p.cu_hist,                                                               \
                     plan, p.Hq, p.Hkv, p.G, p.TC, g, gpart, qcos, p.q_budget, p.nq_pad,      \
                     p.variant, qidx, (void*)(ws + w.gsel), p.kv_budget, sel_idx, kQcosErr,   \
                     (uint64_t*)(ws + w.qkey), (double*)(ws + w.row0))
  const bool mfma = p.dtype == QUOKA_BF16;
  if (p.D == 128) { if (mfma) QUOKA_QSEL(128, true); else QUOKA_QSEL(128, false); }
  else            { if (mfma) QUOKA_QSEL(64, true);  else QUOKA_QSEL(64, false); }
#undef QUOKA_QSEL
  return hipGetLastError();
}

}  // namespace quoka
