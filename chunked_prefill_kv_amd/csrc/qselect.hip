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
// the counters the later kernels accumulate into. Block 0 plans; every block
// clears a slice of [zero_begin, zero_end).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu_chunk,
                                                   const int32_t* __restrict__ cu_hist, int S,
                                                   int32_t* __restrict__ plan,
                                                   uint4* __restrict__ zero, int64_t nzero16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nzero16;
       i += (int64_t)gridDim.x * blockDim.x)
    zero[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    int32_t* qt = plan;
    int32_t* sb = plan + (S + 1);
    int32_t* kt = plan + 2 * (S + 1);
    int32_t a = 0, b = 0, c = 0;
    for (int s = 0; s < S; ++s) {
      qt[s] = a; sb[s] = b; kt[s] = c;
      int C = cu_chunk[s + 1] - cu_chunk[s];
      int L = cu_hist[s + 1] - cu_hist[s];
      a += (C + kQprepTokens - 1) / kQprepTokens;
      b += (L + kScoreKeys - 1) / kScoreKeys;
      c += (L + kTopbKeys - 1) / kTopbKeys;
    }
    qt[S] = a; sb[S] = b; kt[S] = c;
  }
}

hipError_t launch_plan(const Problem& p, char* ws, const Workspace& w, hipStream_t st) {
  int64_t n16 = (int64_t)((w.zero_end - w.zero_begin) / 16);
  int grid = (int)std::min<int64_t>(1024, std::max<int64_t>(1, (n16 + 2047) / 2048));
  hipLaunchKernelGGL(plan_kernel, dim3(grid), dim3(256), 0, st, p.cu_chunk, p.cu_hist, p.S,
                     (int32_t*)(ws + w.plan), (uint4*)(ws + w.zero_begin), n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K1a: g_t = mean_j unit(q_{t,j}) over the G query heads of KV head h, for a
// tile of 64 tokens; also the tile's fp64 sum of g (for the mean query).
// Lanes work in groups of 16 on one head row each (4 rows per instruction).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void qprep_g_kernel(
    const T* __restrict__ q, const int32_t* __restrict__ cu_chunk,
    const int32_t* __restrict__ plan, int S, int Hq, int Hkv, int G, float* __restrict__ g,
    double* __restrict__ gpart) {
  constexpr int EPL = D / 16;  // elements per lane
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* qt_off = plan;
  const int s = upper_seq(qt_off, S, tile);
  const int t0 = (tile - qt_off[s]) * kQprepTokens;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, sub = lane & 15;

  double part[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[e] = 0.0;

  for (int i = 0; i < kQprepTokens / 4; ++i) {
    const int t = t0 + wave * (kQprepTokens / 4) + i;
    if (t >= C) break;  // uniform across the wave
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int j0 = 0; j0 < G; j0 += 4) {
      const int j = j0 + grp;
      float x[EPL];
      if (j < G) {
        const T* row = q + ((int64_t)(c_off + t) * Hq + (int64_t)h * G + j) * D + sub * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = to_f32(row[e]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = 0.f;
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
      const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(x[e], inv, acc[e]);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc[e] += __shfl_xor(acc[e], 16, 64);
      acc[e] += __shfl_xor(acc[e], 32, 64);
      acc[e] /= (float)G;
    }
    if (grp == 0) {
      float* dst = g + ((int64_t)(c_off + t) * Hkv + h) * D + sub * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        dst[e] = acc[e];
        part[e] += (double)acc[e];
      }
    }
  }
  __shared__ double red[4][D];
  if (grp == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[wave][sub * EPL + e] = part[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int i = threadIdx.x;
    gpart[((int64_t)tile * Hkv + h) * D + i] = red[0][i] + red[1][i] + red[2][i] + red[3][i];
  }
}

// ---------------------------------------------------------------------------
// K1b: mean query M of (sequence, KV head) from the tile sums (fixed order,
// fp64), then c_t = cos(M, g_t) for the tile's tokens.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void qprep_cos_kernel(
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TC, const float* __restrict__ g, const double* __restrict__ gpart,
    float* __restrict__ qcos) {
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* qt_off = plan;
  const int s = upper_seq(qt_off, S, tile);
  const int t0 = (tile - qt_off[s]) * kQprepTokens;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ double Md[D];
  __shared__ double red[4];
  double sq = 0.0;
  if (threadIdx.x < D) {
    double acc = 0.0;
    for (int k = qt_off[s]; k < qt_off[s + 1]; ++k)
      acc += gpart[((int64_t)k * Hkv + h) * D + threadIdx.x];
    acc /= (double)C;
    Md[threadIdx.x] = acc;
    sq = acc * acc;
  }
  sq = wave_sum(sq);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  const double mnorm = sqrt(red[0] + red[1] + red[2] + red[3]);

  constexpr int EPL = D / 64;
  double m[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) m[e] = Md[lane * EPL + e];
  for (int i = 0; i < kQprepTokens / 4; ++i) {
    const int t = t0 + wave * (kQprepTokens / 4) + i;
    if (t >= C) break;
    const float* gr = g + ((int64_t)(c_off + t) * Hkv + h) * D + lane * EPL;
    double dot = 0.0, gg = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const double x = (double)gr[e];
      dot += x * m[e];
      gg += x * x;
    }
    dot = wave_sum(dot);
    gg = wave_sum(gg);
    if (lane == 0) {
      const double den = mnorm * sqrt(gg);
      qcos[(int64_t)h * TC + c_off + t] = den > 0.0 ? (float)(dot / den) : 0.f;
    }
  }
}

hipError_t launch_qprep(const Problem& p, const void* q, char* ws, const Workspace& w,
                        float* qcos, hipStream_t st) {
  if (p.NQT == 0) return hipSuccess;
  dim3 grid((unsigned)p.NQT, (unsigned)p.Hkv);
  const int32_t* plan = (const int32_t*)(ws + w.plan);
  float* g = (float*)(ws + w.g);
  double* gpart = (double*)(ws + w.gpart);
#define QUOKA_QPREP(T, D)                                                                    \
  hipLaunchKernelGGL((qprep_g_kernel<T, D>), grid, dim3(256), 0, st, (const T*)q, p.cu_chunk, \
                     plan, p.S, p.Hq, p.Hkv, p.G, g, gpart)
  if (p.dtype == QUOKA_BF16) {
    if (p.D == 128) QUOKA_QPREP(bf16, 128); else QUOKA_QPREP(bf16, 64);
  } else {
    if (p.D == 128) QUOKA_QPREP(float, 128); else QUOKA_QPREP(float, 64);
  }
#undef QUOKA_QPREP
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.D == 128)
    hipLaunchKernelGGL((qprep_cos_kernel<128>), grid, dim3(256), 0, st, p.cu_chunk, plan, p.S,
                       p.Hkv, p.TC, g, gpart, qcos);
  else
    hipLaunchKernelGGL((qprep_cos_kernel<64>), grid, dim3(256), 0, st, p.cu_chunk, plan, p.S,
                       p.Hkv, p.TC, g, gpart, qcos);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K2: per (sequence, KV head) keep the N_q,eff tokens with the lowest cosine
// (ties to the lower token) by an exact radix select over the unique keys
// (order_key(c) << 32 | t), emit them ascending, and lay out the kept g rows
// for the scorer: bf16 hi/lo pairs in MFMA A-operand order, or fp32 rows.
// ---------------------------------------------------------------------------
constexpr int kQselCap = 12288;  // chunk tokens whose cosines are staged in LDS

template <int D, bool kMfma>
__global__ __launch_bounds__(256) void qselect_kernel(
    const int32_t* __restrict__ cu_chunk, int Hkv, int64_t TC, int q_budget, int nq_pad,
    const float* __restrict__ qcos, const float* __restrict__ g, int32_t* __restrict__ qidx,
    void* __restrict__ gsel) {
  const int prob = blockIdx.x;
  const int s = prob / Hkv, h = prob % Hkv;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int n = min(q_budget, C);
  int32_t* out = qidx + (int64_t)prob * q_budget;

  __shared__ float cs[kQselCap];
  __shared__ int32_t kept[QUOKA_MAX_Q_BUDGET];
  __shared__ RadixScratch rs;

  const float* src = qcos + (int64_t)h * TC + c_off;
  if (C <= kQselCap) {
    for (int i = threadIdx.x; i < C; i += blockDim.x) cs[i] = src[i];
    src = cs;
  }
  __syncthreads();

  auto key_of = [&](int t) -> uint64_t {
    return ((uint64_t)float_order_key(src[t]) << 32) | (uint32_t)t;
  };
  uint64_t thr = ~0ull;
  if (n < C) thr = radix_select_kth<false>(key_of, C, n, rs);  // n-th smallest key

  // ascending compaction of the kept tokens
  const int per = (C + blockDim.x - 1) / blockDim.x;
  const int b0 = threadIdx.x * per, b1 = min(C, b0 + per);
  int cnt = 0;
  for (int t = b0; t < b1; ++t) cnt += (key_of(t) <= thr);
  int pos = block_exclusive_scan_256(cnt, rs);
  for (int t = b0; t < b1; ++t) {
    if (key_of(t) <= thr) {
      out[pos] = t;
      kept[pos] = t;
      ++pos;
    }
  }
  for (int i = n + threadIdx.x; i < q_budget; i += blockDim.x) out[i] = -1;
  __syncthreads();
  if (n == 0) return;

  // kept group queries for the scorer
  if constexpr (kMfma) {
    // A operand of v_mfma_f32_16x16x32_bf16: lane l holds row l%16 and the
    // 8 d-values (l/16)*8.. of the 32-wide d-step. Rows past n repeat row 0,
    // which leaves the max over kept tokens unchanged.
    bf16* dst = (bf16*)gsel + (int64_t)prob * nq_pad * D * 2;
    const int total = nq_pad * D * 2;
    for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
      const int e = idx & 7;
      const int lane = (idx >> 3) & 63;
      const int term = (idx >> 9) & 1;
      const int rest = idx >> 10;  // qb * (D/32) + ds
      const int ds = rest % (D / 32), qb = rest / (D / 32);
      const int row = qb * 16 + (lane & 15);
      const int d = ds * 32 + (lane >> 4) * 8 + e;
      const int t = kept[row < n ? row : 0];
      const float x = g[((int64_t)(c_off + t) * Hkv + h) * D + d];
      const bf16 hi = (bf16)x;
      dst[idx] = term == 0 ? hi : (bf16)(x - (float)hi);
    }
  } else {
    float* dst = (float*)gsel + (int64_t)prob * nq_pad * D;
    for (int idx = threadIdx.x; idx < n * D; idx += blockDim.x) {
      const int row = idx / D, d = idx % D;
      dst[idx] = g[((int64_t)(c_off + kept[row]) * Hkv + h) * D + d];
    }
  }
}

hipError_t launch_qselect(const Problem& p, char* ws, const Workspace& w, const float* qcos,
                          int32_t* qidx, hipStream_t st) {
  dim3 grid((unsigned)(p.S * p.Hkv));
  const float* g = (const float*)(ws + w.g);
  void* gsel = ws + w.gsel;
#define QUOKA_QSEL(D, M)                                                                      \
  hipLaunchKernelGGL((qselect_kernel<D, M>), grid, dim3(256), 0, st, p.cu_chunk, p.Hkv, p.TC, \
                     p.q_budget, p.nq_pad, qcos, g, qidx, gsel)
  const bool mfma = p.dtype == QUOKA_BF16;
  if (p.D == 128) { if (mfma) QUOKA_QSEL(128, true); else QUOKA_QSEL(128, false); }
  else            { if (mfma) QUOKA_QSEL(64, true);  else QUOKA_QSEL(64, false); }
#undef QUOKA_QSEL
  return hipGetLastError();
}

}  // namespace quoka
