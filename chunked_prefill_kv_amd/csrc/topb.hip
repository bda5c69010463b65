// K4: exact top-B_eff of the key scores per (sequence, KV head), ties to the
// lower key index, indices written ascending with -1 padding.
// Sources: "QUOKA Explained", "From scores to a smaller KV set" (rank the keys
// and keep the top ones within the sparse-attention budget); QUOKA paper
// summary (hw-hk.tistory.com/367), "Background > Attention Sparsity".
//
// Three launches, all exact:
//   filter : every workgroup re-derives from the scorer's histogram the bin
//            b* that holds the B_eff-th score; keys above b* are in, keys in
//            b* become candidates (score key, index) appended per problem;
//   cands  : one workgroup per problem radix-selects the `need` best
//            candidates (composite key (score key << 32) | ~index, unique) and
//            counts the chosen ones per tile;
//   write  : each tile offsets itself by the counts of the tiles before it and
//            writes its selected indices in ascending order.
#include "common.h"
#include "internal.h"
#include "radix.h"

namespace quoka {

__device__ __forceinline__ uint64_t cand_key(float sc, int key) {
  return ((uint64_t)float_order_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)key);
}

// b*, keys above it and the number still needed from it, for one problem.
// Every thread returns the same values.
__device__ void find_threshold_bin(const uint32_t* __restrict__ h, int L, int B_eff,
                                   RadixScratch& rs, int* bstar, int* above, int* need) {
  __shared__ int sh[3];
  if (B_eff >= L) {
    *bstar = -1; *above = L; *need = 0;
    return;
  }
  // thread i owns bins [kScoreBins - 8(i+1), kScoreBins - 8i): counting from the top
  constexpr int PER = kScoreBins / 256;
  uint32_t c[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    c[e] = h[kScoreBins - 1 - (threadIdx.x * PER + e)];
    tot += c[e];
  }
  uint32_t cum = block_exclusive_scan_256(tot, rs);  // keys in higher bins
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (cum < (uint32_t)B_eff && (uint32_t)B_eff <= cum + c[e]) {
      sh[0] = kScoreBins - 1 - (threadIdx.x * PER + e);
      sh[1] = (int)cum;
      sh[2] = B_eff - (int)cum;
    }
    cum += c[e];
  }
  __syncthreads();
  *bstar = sh[0]; *above = sh[1]; *need = sh[2];
  __syncthreads();
}

__global__ __launch_bounds__(256) void topb_filter_kernel(
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int64_t NKT, int kv_budget, const float* __restrict__ scores,
    const uint32_t* __restrict__ hist, Threshold* __restrict__ thr, uint32_t* __restrict__ ccount,
    uint64_t* __restrict__ cand, uint32_t* __restrict__ gtcount) {
  __shared__ RadixScratch rs;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* kt_off = plan + 2 * (S + 1);
  const int s = upper_seq(kt_off, S, tile);
  const int lt = tile - kt_off[s];
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, L);
  const int prob = s * Hkv + h;

  int bstar, above, need;
  find_threshold_bin(hist + (int64_t)prob * kScoreBins, L, B_eff, rs, &bstar, &above, &need);
  if (lt == 0 && threadIdx.x == 0) {
    Threshold t;
    t.bstar = bstar; t.above = above; t.need = need; t.pad = 0;
    t.prefix = ~0ull; t.mask = ~0ull;
    thr[prob] = t;
  }
  const float* srow = scores + (int64_t)h * TL + h_off;
  uint64_t* crow = cand + (int64_t)h * TL + h_off;
  const int lane = threadIdx.x & 63;
  const int k0 = lt * kTopbKeys;
  constexpr int PER = kTopbKeys / 256;
  float sc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int key = k0 + i * 256 + threadIdx.x;
    sc[i] = key < L ? srow[key] : 0.f;
  }
  uint32_t gt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int key = k0 + i * 256 + threadIdx.x;
    const bool ok = key < L;
    const int bin = score_bin(sc[i]);
    gt += (ok && bin > bstar);
    const bool isc = ok && bin == bstar;
    const uint64_t bal = __ballot(isc);
    if (bal) {  // uniform across the wave
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&ccount[prob], (uint32_t)__popcll(bal));
      base = __shfl(base, 0, 64);
      if (isc) {
        const uint32_t rank = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        crow[base + rank] = cand_key(sc[i], key);
      }
    }
  }
  gt = block_sum_256(gt, rs);
  if (threadIdx.x == 0) gtcount[(int64_t)h * NKT + tile] = gt;
}

__global__ __launch_bounds__(256) void topb_cands_kernel(
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int64_t NKT, int kv_budget, Threshold* __restrict__ thr,
    const uint32_t* __restrict__ ccount, const uint64_t* __restrict__ cand,
    uint32_t* __restrict__ chcount, int32_t* __restrict__ sel_idx) {
  __shared__ RadixScratch rs;
  __shared__ uint64_t lc[kCandCap];
  const int prob = blockIdx.x;
  const int s = prob / Hkv, h = prob % Hkv;
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, L);
  int32_t* out = sel_idx + (int64_t)prob * kv_budget;
  for (int i = B_eff + threadIdx.x; i < kv_budget; i += 256) out[i] = -1;
  if (L == 0) return;
  const Threshold t = thr[prob];
  if (t.bstar < 0 || t.need <= 0) return;
  const int n = (int)ccount[prob];
  const uint64_t* src = cand + (int64_t)h * TL + h_off;
  if (n <= kCandCap) {
    block_copy<256, 8>(lc, src, n);
    src = lc;
  }
  __syncthreads();
  uint64_t prefix = ~0ull, mask = 0ull;  // n == need: every candidate is chosen
  if (t.need < n) radix_select<true>([&](int i) { return src[i]; }, n, t.need, rs, prefix, mask);
  else prefix = 0ull;
  if (threadIdx.x == 0) {
    thr[prob].prefix = prefix;
    thr[prob].mask = mask;
  }
  const int32_t* kt_off = plan + 2 * (S + 1);
  uint32_t* ch = chcount + (int64_t)h * NKT + kt_off[s];
  for (int i = threadIdx.x; i < n; i += 256) {
    const uint64_t c = src[i];
    if (radix_taken<true>(c, prefix, mask)) {
      const int key = (int)(0xFFFFFFFFu - (uint32_t)c);
      atomicAdd(&ch[key / kTopbKeys], 1u);
    }
  }
}

__global__ __launch_bounds__(256) void topb_write_kernel(
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int64_t NKT, int kv_budget, const float* __restrict__ scores,
    const Threshold* __restrict__ thr, const uint32_t* __restrict__ gtcount,
    const uint32_t* __restrict__ chcount, int32_t* __restrict__ sel_idx) {
  __shared__ RadixScratch rs;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* kt_off = plan + 2 * (S + 1);
  const int s = upper_seq(kt_off, S, tile);
  const int lt = tile - kt_off[s];
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int prob = s * Hkv + h;
  const Threshold t = thr[prob];

  uint32_t before = 0;
  for (int i = kt_off[s] + threadIdx.x; i < tile; i += 256)
    before += gtcount[(int64_t)h * NKT + i] + chcount[(int64_t)h * NKT + i];
  before = block_sum_256(before, rs);

  const float* srow = scores + (int64_t)h * TL + h_off;
  constexpr int PER = kTopbKeys / 256;
  const int k0 = lt * kTopbKeys + threadIdx.x * PER;
  uint32_t flags = 0, cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int key = k0 + e;
    if (key < L) {
      const float sc = srow[key];
      const int bin = score_bin(sc);
      const bool sel = bin > t.bstar ||
                       (bin == t.bstar && radix_taken<true>(cand_key(sc, key), t.prefix, t.mask));
      flags |= (uint32_t)sel << e;
      cnt += sel;
    }
  }
  uint32_t pos = before + block_exclusive_scan_256(cnt, rs);
  int32_t* out = sel_idx + (int64_t)prob * kv_budget;
  const uint32_t b_eff = (uint32_t)min(kv_budget, L);
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if ((flags & (1u << e)) && pos < b_eff) out[pos++] = k0 + e;
}

hipError_t launch_topb(const Problem& p, char* ws, const Workspace& w, const float* scores,
                       int32_t* sel_idx, hipStream_t st) {
  const int32_t* plan = (const int32_t*)(ws + w.plan);
  Threshold* thr = (Threshold*)(ws + w.thr);
  uint32_t* ccount = (uint32_t*)(ws + w.ccount);
  uint64_t* cand = (uint64_t*)(ws + w.cand);
  uint32_t* gtc = (uint32_t*)(ws + w.gtcount);
  uint32_t* chc = (uint32_t*)(ws + w.chcount);
  const uint32_t* hist = (const uint32_t*)(ws + w.hist);
  if (p.NKT > 0) {
    hipLaunchKernelGGL(topb_filter_kernel, dim3((unsigned)p.NKT, (unsigned)p.Hkv), dim3(256), 0,
                       st, p.cu_hist, plan, p.S, p.Hkv, p.TL, p.NKT, p.kv_budget, scores, hist,
                       thr, ccount, cand, gtc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(topb_cands_kernel, dim3((unsigned)(p.S * p.Hkv)), dim3(256), 0, st,
                     p.cu_hist, plan, p.S, p.Hkv, p.TL, p.NKT, p.kv_budget, thr, ccount, cand,
                     chc, sel_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.NKT == 0) return e;
  hipLaunchKernelGGL(topb_write_kernel, dim3((unsigned)p.NKT, (unsigned)p.Hkv), dim3(256), 0, st,
                     p.cu_hist, plan, p.S, p.Hkv, p.TL, p.NKT, p.kv_budget, scores, thr, gtc, chc,
                     sel_idx);
  return hipGetLastError();
}

}  // namespace quoka
