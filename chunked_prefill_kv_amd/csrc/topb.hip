// K4: exact top-B_eff of the key scores per (sequence, KV head), ties to the
// lower key index, indices written ascending with -1 padding.
// Sources: "QUOKA Explained", "From scores to a smaller KV set" (rank the keys
// and keep the top ones within the sparse-attention budget); QUOKA paper
// summary (hw-hk.tistory.com/367), "Background > Attention Sparsity".
//
// Three launches, all exact:
//   filter : every workgroup derives from the scorer's histogram the bin b*
//            holding the B_eff-th score; keys above b* are in, keys in b*
//            become candidates (composite key (score key << 32) | ~index,
//            unique) appended per problem (one global atomic per workgroup);
//   cands  : one workgroup per problem radix-selects the `need` best
//            candidates and counts the chosen ones per tile;
//   write  : each tile offsets itself by the counts of the tiles before it and
//            writes its selected indices in ascending order.
#include "common.h"
#include "internal.h"
#include "radix.h"

namespace quoka {

__device__ __forceinline__ uint64_t cand_key(float sc, int key) {
  return ((uint64_t)float_order_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)key);
}

// The histogram's bin function: linear over [-1, 1], or over all floats for
// the unbounded dot-product scores (kRaw).
template <bool kRaw>
__device__ __forceinline__ int bin_of(float s) {
  return kRaw ? score_bin_raw(s) : score_bin(s);
}

// Keys above the threshold bin b* are counted per tile; keys inside b* are
// appended to the problem's candidate list (one global atomic per workgroup).
// Tile 0 of each problem records b* for the later launches.
template <bool kRaw>
__global__ __launch_bounds__(256) void topb_filter_kernel(
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int64_t NKT, const float* __restrict__ scores, Threshold* __restrict__ thr,
    uint32_t* __restrict__ ccount, uint64_t* __restrict__ cand, uint32_t* __restrict__ gtcount,
    const uint32_t* __restrict__ hist, int kv_budget) {
  __shared__ RadixScratch<256> rs;
  __shared__ uint32_t wcnt[4], wbase[4];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* kt_off = plan + 2 * (S + 1);
  const int s = upper_seq(kt_off, S, tile);
  const int lt = tile - kt_off[s];
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int prob = s * Hkv + h;
  // the tile's scores are requested before the threshold search over the
  // histogram, so the two latencies overlap
  const float* srow = scores + (int64_t)h * TL + h_off;
  uint64_t* crow = cand + (int64_t)h * TL + h_off;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = lt * kTopbKeys;
  constexpr int PER = kTopbKeys / 256;
  float sc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int key = k0 + i * 256 + threadIdx.x;
    sc[i] = key < L ? srow[key] : 0.f;
  }
  Threshold t;
  find_threshold_bin<256>(hist + (int64_t)prob * kScoreBins, L, min(kv_budget, L), rs, &t.bstar,
                          &t.above, &t.need);
  uint32_t gt = 0, nc = 0;
  uint64_t bal[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int key = k0 + i * 256 + threadIdx.x;
    const bool ok = key < L;
    const int bin = bin_of<kRaw>(sc[i]);
    gt += (ok && bin > t.bstar);
    bal[i] = __ballot(ok && bin == t.bstar);
    nc += (uint32_t)__popcll(bal[i]);
  }
  if (lane == 0) wcnt[wave] = nc;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t tot = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    uint32_t b = tot ? atomicAdd(&ccount[prob], tot) : 0u;
    for (int w = 0; w < 4; ++w) { wbase[w] = b; b += wcnt[w]; }
  }
  __syncthreads();
  uint32_t base = wbase[wave];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (bal[i] >> lane & 1ull) {
      const uint32_t rank = (uint32_t)__popcll(bal[i] & ((1ull << lane) - 1ull));
      crow[base + rank] = cand_key(sc[i], k0 + i * 256 + (int)threadIdx.x);
    }
    base += (uint32_t)__popcll(bal[i]);
  }
  gt = block_sum<256>(gt, rs);
  if (threadIdx.x == 0) gtcount[(int64_t)h * NKT + tile] = gt;

  if (lt == 0 && threadIdx.x == 0) { t.prefix = ~0ull; t.mask = ~0ull; thr[prob] = t; }
}

// One workgroup per problem: the `need` best candidates of bin b*, exactly,
// and the count of chosen candidates per tile.
__global__ __launch_bounds__(256) void topb_cands_kernel(
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int64_t NKT, Threshold* __restrict__ thr, const uint32_t* __restrict__ ccount,
    const uint64_t* __restrict__ cand, uint32_t* __restrict__ chcount) {
  __shared__ RadixScratch<256> rs;
  const int prob = blockIdx.x, s = prob / Hkv, h = prob % Hkv;
  const int32_t* kt_off = plan + 2 * (S + 1);
  const int h_off = cu_hist[s];
  if (cu_hist[s + 1] == h_off) return;
  Threshold t = thr[prob];
  if (t.bstar < 0 || t.need <= 0) return;
  __shared__ uint64_t lc[kCandCap];
  const int n = (int)ccount[prob];
  const uint64_t* src = cand + (int64_t)h * TL + h_off;
  if (n <= kCandCap) {
    block_copy<256, 8>(lc, src, n);
    src = lc;
  }
  __syncthreads();
  uint64_t prefix = 0ull, mask = 0ull;  // n == need: every candidate is chosen
  if (t.need < n)
    radix_select<true, 256>([&](int i) { return src[i]; }, n, t.need, rs, prefix, mask);
  if (threadIdx.x == 0) {
    t.prefix = prefix;
    t.mask = mask;
    thr[prob] = t;
  }
  // Chosen candidates per tile, counted in LDS (this workgroup owns every
  // tile of its problem) and stored once per tile: device-scope atomics would
  // serialise on the few tile counters when the threshold bin is crowded.
  // Blocks of kTileBlock tiles bound the LDS for any history length.
  constexpr int kTileBlock = 1024;
  __shared__ uint32_t tcnt[kTileBlock];
  uint32_t* ch = chcount + (int64_t)h * NKT + kt_off[s];
  const int ntile = kt_off[s + 1] - kt_off[s];
  for (int t0 = 0; t0 < ntile; t0 += kTileBlock) {
    const int nt = min(kTileBlock, ntile - t0);
    for (int i = threadIdx.x; i < nt; i += 256) tcnt[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) {
      const uint64_t c = src[i];
      if (radix_taken<true>(c, prefix, mask)) {
        const int tl = (int)(0xFFFFFFFFu - (uint32_t)c) / kTopbKeys - t0;
        if (tl >= 0 && tl < nt) atomicAdd(&tcnt[tl], 1u);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt; i += 256) ch[t0 + i] = tcnt[i];
    __syncthreads();
  }
}

template <bool kRaw>
__global__ __launch_bounds__(256) void topb_write_kernel(
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ plan, int S, int Hkv,
    int64_t TL, int64_t NKT, int kv_budget, const float* __restrict__ scores,
    const Threshold* __restrict__ thr, const uint32_t* __restrict__ gtcount,
    const uint32_t* __restrict__ chcount, int32_t* __restrict__ sel_idx) {
  __shared__ RadixScratch<256> rs;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* kt_off = plan + 2 * (S + 1);
  const int s = upper_seq(kt_off, S, tile);
  const int lt = tile - kt_off[s];
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int prob = s * Hkv + h;
  const Threshold t = thr[prob];
  // the tile's scores are requested before the count of the tiles before it
  const float* srow = scores + (int64_t)h * TL + h_off;
  constexpr int PER = kTopbKeys / 256;
  const int k0 = lt * kTopbKeys + threadIdx.x * PER;
  float scv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) scv[e] = k0 + e < L ? srow[k0 + e] : 0.f;

  uint32_t before = 0;
  for (int i = kt_off[s] + threadIdx.x; i < tile; i += 256)
    before += gtcount[(int64_t)h * NKT + i] + chcount[(int64_t)h * NKT + i];
  before = block_sum<256>(before, rs);

  uint32_t flags = 0, cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int key = k0 + e;
    if (key < L) {
      const float sc = scv[e];
      const int bin = bin_of<kRaw>(sc);
      const bool sel = bin > t.bstar ||
                       (bin == t.bstar && radix_taken<true>(cand_key(sc, key), t.prefix, t.mask));
      flags |= (uint32_t)sel << e;
      cnt += sel;
    }
  }
  uint32_t pos = before + block_exclusive_scan<256>(cnt, rs);
  int32_t* out = sel_idx + (int64_t)prob * kv_budget;
  const uint32_t b_eff = (uint32_t)min(kv_budget, L);
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if ((flags & (1u << e)) && pos < b_eff) out[pos++] = k0 + e;
}

hipError_t launch_topb(const Problem& p, char* ws, const Workspace& w, const float* scores,
                       int32_t* sel_idx, hipStream_t st) {
  if (p.NKT == 0) return hipSuccess;
  const int32_t* plan = (const int32_t*)(ws + w.plan);
  Threshold* thr = (Threshold*)(ws + w.thr);
  uint32_t* ccount = (uint32_t*)(ws + w.ccount);
  uint64_t* cand = (uint64_t*)(ws + w.cand);
  uint32_t* gtc = (uint32_t*)(ws + w.gtcount);
  uint32_t* chc = (uint32_t*)(ws + w.chcount);
  const dim3 grid((unsigned)p.NKT, (unsigned)p.Hkv);
  const bool raw = p.mode() == kModeDot;
  if (raw)
    hipLaunchKernelGGL(topb_filter_kernel<true>, grid, dim3(256), 0, st, p.cu_hist, plan, p.S,
                       p.Hkv, p.TL, p.NKT, scores, thr, ccount, cand, gtc,
                       (const uint32_t*)(ws + w.hist), p.kv_budget);
  else
    hipLaunchKernelGGL(topb_filter_kernel<false>, grid, dim3(256), 0, st, p.cu_hist, plan, p.S,
                       p.Hkv, p.TL, p.NKT, scores, thr, ccount, cand, gtc,
                       (const uint32_t*)(ws + w.hist), p.kv_budget);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topb_cands_kernel, dim3((unsigned)(p.S * p.Hkv)), dim3(256), 0, st, p.cu_hist,
                     plan, p.S, p.Hkv, p.TL, p.NKT, thr, ccount, cand, chc);
  if (raw)
    hipLaunchKernelGGL(topb_write_kernel<true>, grid, dim3(256), 0, st, p.cu_hist, plan, p.S,
                       p.Hkv, p.TL, p.NKT, p.kv_budget, scores, thr, gtc, chc, sel_idx);
  else
    hipLaunchKernelGGL(topb_write_kernel<false>, grid, dim3(256), 0, st, p.cu_hist, plan, p.S,
                       p.Hkv, p.TL, p.NKT, p.kv_budget, scores, thr, gtc, chc, sel_idx);
  return hipGetLastError();
}

}  // namespace quoka
