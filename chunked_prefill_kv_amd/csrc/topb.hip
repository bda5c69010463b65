// K4: top-B_eff of the key scores per (sequence, KV head), ties to the lower
// key index, indices written ascending with -1 padding. The kept set is the
// one the fp64 scores define.
// Sources: "QUOKA Explained", "From scores to a smaller KV set" (rank the keys
// and keep the top ones within the sparse-attention budget); QUOKA paper
// summary (hw-hk.tistory.com/367), "Background > Attention Sparsity", and
// "Scoring via Cosine Similarity" / "Aggregation Across Queries and KV Groups"
// for the score the fp64 evaluation computes.
//
// The scorer's fp32 scores are within eps of the fp64 ones (eps bounds its
// rounding, see score_bounds). With s_B the B_eff-th fp32 score, every key
// more than 2 eps above s_B is kept and every key more than 2 eps below it is
// not, whatever the rounding; only the keys between need their fp64 score.
//
// Three launches:
//   filter : every workgroup derives from the scorer's histogram the bin b*
//            holding s_B; the candidate window [lo, hi] is b*'s score range
//            widened by 2 eps on each side, so it holds every key within
//            2 eps of s_B; keys above hi are in and counted per tile; the keys
//            of its tile inside the window are scored in fp64 and stored, as
//            unique keys (fp64 value, then lower index first), at the tile's
//            own offset of the candidate list;
//   cands  : one workgroup per problem: the tiles' candidates gathered, radix
//            select of the B_eff - (keys above hi) best; the chosen ones are
//            marked in a bitmap and counted per tile;
//   write  : each tile offsets itself by the counts of the tiles before it and
//            writes its kept indices (above hi, or marked) ascending.
// The dot-product baseline's scores carry no such bound (they are not
// normalised): its window is the single bin b* and its candidates keep their
// fp32 scores.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "radix.h"

namespace quoka {

__device__ __forceinline__ uint64_t cand_key(float sc, int key) {
  return ((uint64_t)float_order_key(sc) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)key);
}
__device__ __forceinline__ int cand_index(uint64_t c) {
  return (int)(0xFFFFFFFFu - (uint32_t)c);
}

// The histogram's bin function: linear over [-1, 1], or over all floats for
// the unbounded dot-product scores (kRaw).
template <bool kRaw>
__device__ __forceinline__ int bin_of(float s) {
  return kRaw ? score_bin_raw(s) : score_bin(s);
}

// ---------------------------------------------------------------------------
// fp64 scores. For history key k of KV head h the score is max over the kept
// rows r of R_r . k / |k|, where R_r is, per selection:
//   QUOKA, GLOBAL, PER_HEAD   g_t = (1/G) sum_j unit(q_{t,j}) of kept token t,
//                             evaluated as (1/G) sum_j (q_{t,j} . k) / |q_{t,j}|
//   MEAN_QUERIES              the mean of those over the kept tokens (one row)
//   MEAN_QUERY                the chunk's mean query M (one row)
// (the one row comes from the query select, in fp64). A row can hold the max
// only if its fp32 product is within 2 eps_row |k| of the best fp32 product,
// so only those rows are evaluated in fp64: the products of up to 64 keys
// with every kept row are first taken on the MFMA from the scorer's own bf16
// hi/lo rows (fp32 path: every row is evaluated in fp64).
// ---------------------------------------------------------------------------
constexpr int kExactBatch = 64;  // keys per pass (4 key blocks of 16)

struct TopbArgs {
  const int32_t* cu_chunk;
  const int32_t* cu_hist;
  const int32_t* plan;
  int S, Hq, Hkv, G;
  int64_t TL, NKT;
  int kv_budget;
  double eps;              // |fp32 score - fp64 score| <= eps
  const float* scores;
  const uint32_t* hist;
  Threshold* thr;
  uint64_t* cand;          // [Hkv, TL]: tile t's candidates at its own keys' offsets
  uint32_t* ctcount;       // [Hkv, NKT] candidates per tile
  uint32_t* gtcount;
  uint32_t* chcount;
  uint32_t* bits;          // chosen candidates, bit h * TL + cu_hist[s] + key
  float eps_row;           // |fp32 product - fp64 product| <= eps_row |k| per head row
  const void* q;
  const void* k_hist;
  const int32_t* qidx;     // [S, Hkv, q_budget] kept chunk tokens
  int q_budget, nq_pad, variant;
  const double* row0;      // [S, Hkv, D] the one-row baselines' row in fp64
  const void* gsel;        // the scorer's rows (bf16 hi/lo in MFMA order)
};

template <typename T, int D>
struct ExactScratch {
  static constexpr int kCpr = D * (int)sizeof(T) / 16;  // 16-byte pieces per key row
  double knorm2[kExactBatch];
  double lim[kExactBatch];              // least fp32 product of a row that can hold the max
  unsigned long long kmax[kExactBatch]; // order key of the best fp64 product
  int kidx[kExactBatch];
  uint32_t smax[kExactBatch];           // order key of the best fp32 product
  uint32_t npairs;
  uint16_t pairs[kExactBatch * QUOKA_MAX_Q_BUDGET];  // key (6 bits) << 8 | row (7 bits)
  uint4 krows[kExactBatch][kCpr];                    // the batch's key rows
  double row0[D];
};

// A operands of the MFMA screening for the wave's row blocks w and w + 4
// (hi and lo terms per d-step); loaded by the filter before its threshold
// search, so that their latency overlaps it.
template <int D>
struct ScreenRows {
  static constexpr int NDS = D / 32;
  bf16x8 a[2][NDS][2];
};

template <int D>
__device__ __forceinline__ void load_screen_rows(const bf16x8* __restrict__ gs, int nqb, int GH,
                                                 int jh, ScreenRows<D>& sr) {
  constexpr int NDS = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qb = wave + 4 * j;
    if (qb < nqb) {
      const bf16x8* la = gs + (qb * GH + jh) * NDS * 2 * 64 + lane;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        sr.a[j][ds][0] = la[(ds * 2 + 0) * 64];
        sr.a[j][ds][1] = la[(ds * 2 + 1) * 64];
      }
    }
  }
}

// Exact keys exact_key_desc(fp64 score, position) of the history positions
// keys[0..nk) of sequence s, KV head h, into out[0..nk), by one workgroup of
// 256 threads. The batch's key rows are staged in LDS once; products are
// taken by quads (four lanes per key or per (key, row) pair, D / 4 elements
// each). pre: the screening rows of the first batch, already loaded.
template <typename T, int D>
__device__ void exact_keys(const TopbArgs& a, int s, int h, const int* __restrict__ keys,
                           int nk_all, uint64_t* __restrict__ out, ExactScratch<T, D>& xs,
                           ScreenRows<D>& pre, bool have_pre) {
  constexpr int NDS = D / 32;
  constexpr int QE = D / 4;  // elements per lane of a quad
  constexpr int CPR = ExactScratch<T, D>::kCpr;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int HB = 2;                     // query heads in flight per pair
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int quad = threadIdx.x >> 2, ql = threadIdx.x & 3;
  const int prob = s * a.Hkv + h;
  const int c_off = a.cu_chunk[s];
  const int C = a.cu_chunk[s + 1] - c_off;
  const int h_off = a.cu_hist[s];
  const T* q = (const T*)a.q;
  const T* kh = (const T*)a.k_hist;
  const bool one = a.variant == QUOKA_VARIANT_MEAN_QUERIES || a.variant == QUOKA_VARIANT_MEAN_QUERY;
  const int GH = a.variant == QUOKA_VARIANT_PER_HEAD ? a.G : 1;
  const int nrows = C == 0 ? 0 : one ? 1 : min(a.q_budget, C);
  const int32_t* kept = a.qidx + (int64_t)prob * a.q_budget;
  // LDS slot of 16-byte piece c of batch key i's row: bf16 rows are stored
  // with their pieces permuted (c ^ (i & 15) for d = 128, c ^ ((i >> 1) & 7)
  // for d = 64) so that the screen's B-operand reads, one piece of 16 rows
  // per 16 lanes, hit distinct banks
  auto kslot = [](int i, int c) -> int {
    if constexpr (sizeof(T) != 2) return c;
    else return c ^ (D == 128 ? (i & 15) : ((i >> 1) & 7));
  };
  // element e of the LDS row of batch key i
  auto kel = [&](int i, int e) -> double {
    const T* row = (const T*)&xs.krows[i][kslot(i, e / EPC)];
    return (double)to_f32(row[e % EPC]);
  };
  if (one && nrows > 0)
    for (int d = threadIdx.x; d < D; d += 256) xs.row0[d] = a.row0[(int64_t)prob * D + d];

  for (int b0 = 0; b0 < nk_all; b0 += kExactBatch) {
    const int nk = min(kExactBatch, nk_all - b0);
    if (threadIdx.x < kExactBatch) {
      const int i = threadIdx.x;
      xs.kmax[i] = 0ull;  // below the order key of every double
      xs.smax[i] = 0u;
      xs.kidx[i] = i < nk ? keys[b0 + i] : keys[b0];  // keys past nk repeat the first
    }
    if (threadIdx.x == 0) xs.npairs = 0u;
    __syncthreads();
    for (int c = threadIdx.x; c < kExactBatch * CPR; c += 256) {
      const int i = c / CPR, pc = c - i * CPR;
      const T* row = kh + ((int64_t)(h_off + xs.kidx[i]) * a.Hkv + h) * D;
      xs.krows[i][kslot(i, pc)] = *(const uint4*)(row + pc * EPC);
    }
    __syncthreads();
    // |k|^2 in fp64 (exact products of bf16 values), quad i for key i
    if (quad < nk) {
      double ss = 0.0;
#pragma unroll 8
      for (int e = 0; e < QE; ++e) {
        const double x = kel(quad, ql * QE + e);
        ss = fma(x, x, ss);
      }
      ss = quad_sum(ss);
      if (ql == 0) xs.knorm2[quad] = ss;
    }

    // rows that can hold each key's max
    if constexpr (sizeof(T) == 2) {
      if (nrows > 1) {
        // fp32 products on the MFMA: wave w takes the 16-row blocks w and
        // w + 4 (at most 8 blocks) against all 64 keys of the batch, and
        // keeps them in registers
        const int nqb = (nrows + 15) / 16;
        const bf16x8* gs = (const bf16x8*)a.gsel + (int64_t)prob * (a.nq_pad / 16) * GH * NDS * 2 * 64;
        f32x4 acc[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[j][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int jh = 0; jh < GH; ++jh) {
          // the rows of head row jh (the prefetched ones serve the first batch)
          if (!(have_pre && b0 == 0 && jh == 0)) load_screen_rows<D>(gs, nqb, GH, jh, pre);
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) {
            // B operand (keys): lane l reads key c*16 + l%16, d-values (l/16)*8 of step ds
            bf16x8 kb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
              kb[c] = __builtin_bit_cast(bf16x8, xs.krows[c * 16 + (lane & 15)][kslot(c * 16 + (lane & 15), ds * 4 + (lane >> 4))]);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              if (wave + 4 * j < nqb) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  acc[j][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pre.a[j][ds][0], kb[c], acc[j][c], 0, 0, 0);
                  acc[j][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pre.a[j][ds][1], kb[c], acc[j][c], 0, 0, 0);
                }
              }
            }
          }
        }
        // lane l holds rows qb*16 + (l>>4)*4 + e of key column l & 15
        const int rl0 = wave * 16 + (lane >> 4) * 4;  // this lane's first row
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint32_t best = 0u;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (rl0 + 64 * j + e < nrows) best = max(best, float_order_key(acc[j][c][e]));
          const int i = c * 16 + (lane & 15);
          if (i < nk) atomicMax(&xs.smax[i], best);
        }
        __syncthreads();
        if (threadIdx.x < nk) {
          const int i = threadIdx.x;
          xs.lim[i] = (double)float_from_order_key(xs.smax[i]) -
                      2.0 * (double)a.eps_row * (double)GH * sqrt(xs.knorm2[i]);
        }
        __syncthreads();
        const int rl = wave * 16 + (lane >> 4) * 4;  // this lane's first row
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = c * 16 + (lane & 15);
          const double lim = i < nk ? xs.lim[i] : INFINITY;
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if ((double)acc[j][c][e] >= lim && rl + 64 * j + e < nrows)
                xs.pairs[atomicAdd(&xs.npairs, 1u)] = (uint16_t)((i << 8) | (rl + 64 * j + e));
            }
        }
      } else {
        for (int v = threadIdx.x; v < nk * nrows; v += 256) xs.pairs[v] = (uint16_t)(v << 8);
        if (threadIdx.x == 0) xs.npairs = (uint32_t)(nk * nrows);
      }
    } else {
      for (int v = threadIdx.x; v < nk * nrows; v += 256) {
        const int i = v / nrows, r = v - i * nrows;
        xs.pairs[v] = (uint16_t)((i << 8) | r);
      }
      if (threadIdx.x == 0) xs.npairs = (uint32_t)(nk * nrows);
    }
    __syncthreads();

    // fp64 products of the candidate (key, row) pairs, eight lanes each
    // (D / 8 elements per lane)
    {
      constexpr int OE = D / 8, OL = OE / 8;
      const int oct = threadIdx.x >> 3, ol = threadIdx.x & 7;
      const int np = (int)xs.npairs;
      for (int p0 = 0; p0 < np; p0 += 32) {
        const int p = p0 + oct;
        if (p < np) {  // uniform over the eight lanes
          const uint32_t pr = xs.pairs[p];
          const int i = (int)(pr >> 8), r = (int)(pr & 255u);
          Raw8<T> kr[OL];  // this lane's slice of the key, in its storage type
#pragma unroll
          for (int u = 0; u < OL; ++u) {
            // 8 elements: one piece (bf16), or two consecutive ones (fp32, unpermuted)
            const int e0 = ol * OE + u * 8;
            kr[u].load((const T*)&xs.krows[i][kslot(i, e0 / EPC)] + e0 % EPC);
          }
          double dot = 0.0;
          if (one) {
#pragma unroll
            for (int u = 0; u < OL; ++u)
#pragma unroll
              for (int e = 0; e < 8; ++e) dot = fma(xs.row0[ol * OE + u * 8 + e], kr[u][e], dot);
            dot = oct_sum(dot);
          } else {
            // (1/G) sum_j (q_j . k) / |q_j| over the kept token's query heads
            const T* qt = q + ((int64_t)(c_off + kept[r]) * a.Hq + (int64_t)h * a.G) * D + ol * OE;
            for (int j0 = 0; j0 < a.G; j0 += HB) {
              Raw8<T> x[HB][OL];
#pragma unroll
              for (int jj = 0; jj < HB; ++jj)
                if (j0 + jj < a.G)
#pragma unroll
                  for (int u = 0; u < OL; ++u) x[jj][u].load(qt + (int64_t)(j0 + jj) * D + u * 8);
#pragma unroll
              for (int jj = 0; jj < HB; ++jj) {
                if (j0 + jj < a.G) {
                  double xk = 0.0, xx = 0.0;
#pragma unroll
                  for (int u = 0; u < OL; ++u)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                      const double xv = x[jj][u][e];
                      xk = fma(xv, kr[u][e], xk);
                      xx = fma(xv, xv, xx);
                    }
                  xk = oct_sum(xk);
                  xx = oct_sum(xx);
                  if (xx > 0.0) dot += xk / sqrt(xx);
                }
              }
            }
            dot /= (double)a.G;
          }
          if (ol == 0) atomicMax(&xs.kmax[i], (unsigned long long)double_order_key(dot));
        }
      }
    }
    __syncthreads();
    if (threadIdx.x < nk) {
      const int i = threadIdx.x;
      double sc = 0.0;
      if (nrows > 0 && xs.knorm2[i] > 0.0)
        sc = double_from_order_key(xs.kmax[i]) / sqrt(xs.knorm2[i]);
      out[b0 + i] = exact_key_desc(sc, xs.kidx[i]);
    }
    __syncthreads();
  }
}

// Keys above the candidate window are counted per tile; keys inside it are
// stored at the tile's own offset of the problem's candidate list (fp64
// scores unless kRaw) and counted. Tile 0 of each problem records the
// threshold for the later launches.
template <typename T, int D, bool kRaw>
__global__ __launch_bounds__(256, 2) void topb_filter_kernel(const TopbArgs a) {
  __shared__ RadixScratch<256> rs;
  __shared__ uint32_t wcnt[4];
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* kt_off = a.plan + 2 * (a.S + 1);
  const int s = upper_seq(kt_off, a.S, tile);
  const int lt = tile - kt_off[s];
  const int h_off = a.cu_hist[s];
  const int L = a.cu_hist[s + 1] - h_off;
  const int prob = s * a.Hkv + h;
  // the tile's scores (and the screening rows) are requested before the
  // threshold search over the histogram, so the latencies overlap
  const float* srow = a.scores + (int64_t)h * a.TL + h_off;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int k0 = lt * kTopbKeys;
  uint64_t* crow = a.cand + (int64_t)h * a.TL + h_off + k0;
  constexpr int PER = kTopbKeys / 256;
  // unconditional loads (indices clamped into the sequence, L >= 1 here), so
  // that all of them are in flight at once
  float sc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sc[i] = srow[min(k0 + i * 256 + (int)threadIdx.x, L - 1)];
  ScreenRows<D> pre;
  bool have_pre = false;
  if constexpr (!kRaw && sizeof(T) == 2) {
    const int C = a.cu_chunk[s + 1] - a.cu_chunk[s];
    const int nrows = min(a.q_budget, C);
    if (a.variant != QUOKA_VARIANT_MEAN_QUERIES && a.variant != QUOKA_VARIANT_MEAN_QUERY &&
        nrows > 1) {
      const int GH = a.variant == QUOKA_VARIANT_PER_HEAD ? a.G : 1;
      const bf16x8* gs = (const bf16x8*)a.gsel + (int64_t)prob * (a.nq_pad / 16) * GH * (D / 32) * 2 * 64;
      load_screen_rows<D>(gs, (nrows + 15) / 16, GH, 0, pre);
      have_pre = true;
    }
  }
  const uint32_t* hp = a.hist + (int64_t)prob * kScoreBins;
  const int b_eff = min(a.kv_budget, L);
  Threshold t;
  {
    int above, need;
    find_threshold_bin<256>(hp, L, b_eff, rs, &t.bstar, &above, &need);
  }
  t.pad = 0;
  // the window: kRaw, the bin b* itself; else b*'s score range (a score s
  // lands in bin floor(fp32(s + 1) * 1024), fp32(s + 1) within 2^-23 of
  // s + 1) widened by 2 eps on each side
  t.lo = (double)t.bstar / (kScoreBins / 2) - 1.0 - 0x1p-22 - 2.0 * a.eps;
  t.hi = (double)(t.bstar + 1) / (kScoreBins / 2) - 1.0 + 0x1p-22 + 2.0 * a.eps;
  uint32_t gt = 0, nc = 0;
  uint64_t bal[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int key = k0 + i * 256 + threadIdx.x;
    const bool ok = key < L && t.bstar >= 0;
    bool above, cand;
    if constexpr (kRaw) {
      const int bin = bin_of<true>(sc[i]);
      above = bin > t.bstar;
      cand = bin == t.bstar;
    } else {
      const double v = (double)sc[i];
      above = v > t.hi;
      cand = v >= t.lo && !above;
    }
    gt += (ok && above);
    bal[i] = __ballot(ok && cand);
    nc += (uint32_t)__popcll(bal[i]);
  }
  if (lane == 0) wcnt[wave] = nc;
  gt = block_sum<256>(gt, rs);  // its barriers also publish wcnt
  const uint32_t tot = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  if (threadIdx.x == 0) {
    a.gtcount[(int64_t)h * a.NKT + tile] = gt;
    a.ctcount[(int64_t)h * a.NKT + tile] = tot;
    if (lt == 0) a.thr[prob] = t;
  }
  uint32_t base = 0u;
  for (int w = 0; w < wave; ++w) base += wcnt[w];
  if constexpr (kRaw) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (bal[i] >> lane & 1ull) {
        const uint32_t rank = (uint32_t)__popcll(bal[i] & ((1ull << lane) - 1ull));
        crow[base + rank] = cand_key(sc[i], k0 + i * 256 + (int)threadIdx.x);
      }
      base += (uint32_t)__popcll(bal[i]);
    }
  } else {
    // the tile's candidates, scored in fp64
    __shared__ int ckey[kTopbKeys];
    __shared__ ExactScratch<T, D> xs;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (bal[i] >> lane & 1ull) {
        const uint32_t rank = (uint32_t)__popcll(bal[i] & ((1ull << lane) - 1ull));
        ckey[base + rank] = k0 + i * 256 + (int)threadIdx.x;
      }
      base += (uint32_t)__popcll(bal[i]);
    }
    __syncthreads();
    if (tot) exact_keys<T, D>(a, s, h, ckey, (int)tot, crow, xs, pre, have_pre);
  }
}

// One workgroup per problem: the problem's candidates gathered from its
// tiles, the `need` best of them, marked in the bitmap and counted per tile.
template <bool kRaw>
__global__ __launch_bounds__(256) void topb_cands_kernel(const TopbArgs a) {
  __shared__ RadixScratch<256> rs;
  __shared__ uint64_t lc[kCandCap];
  const int prob = blockIdx.x, s = prob / a.Hkv, h = prob % a.Hkv;
  const int32_t* kt_off = a.plan + 2 * (a.S + 1);
  const int h_off = a.cu_hist[s];
  const int L = a.cu_hist[s + 1] - h_off;
  if (L == 0) return;
  const Threshold t = a.thr[prob];
  if (t.bstar < 0) return;  // every key is kept
  const int ntile = kt_off[s + 1] - kt_off[s];
  const uint32_t* ctc = a.ctcount + (int64_t)h * a.NKT + kt_off[s];
  const uint32_t* gtc = a.gtcount + (int64_t)h * a.NKT + kt_off[s];
  const uint64_t* crow = a.cand + (int64_t)h * a.TL + h_off;
  uint32_t n = 0u, above = 0u;
  for (int i = threadIdx.x; i < ntile; i += 256) {
    n += ctc[i];
    above += gtc[i];
  }
  n = block_sum<256>(n, rs);
  above = block_sum<256>(above, rs);
  const int need = min(a.kv_budget, L) - (int)above;  // 1 <= need <= n
  // Gathered 256 tiles at a time: their offsets by a scan, then every thread
  // copies entries (finding each one's tile by a binary search over the
  // offsets), so that the loads are all in flight together. Past the LDS the
  // candidates are compacted in place to the front of the problem's list:
  // entry i comes from position >= i, so 256 entries at a time are read into
  // registers and written after a barrier.
  const bool in_lds = n <= (uint32_t)kCandCap;
  uint64_t* dst = in_lds ? lc : a.cand + (int64_t)h * a.TL + h_off;
  __shared__ uint32_t toff[257];
  uint32_t base = 0u;
  for (int t0 = 0; t0 < ntile; t0 += 256) {
    const int nt = min(256, ntile - t0);
    const uint32_t c = (int)threadIdx.x < nt ? ctc[t0 + threadIdx.x] : 0u;
    const uint32_t excl = block_exclusive_scan<256>(c, rs);
    toff[threadIdx.x] = excl;
    if (threadIdx.x == 255) toff[256] = excl + c;
    __syncthreads();
    const uint32_t m = toff[256];
    for (uint32_t i0 = 0; i0 < m; i0 += 256) {
      const uint32_t i = i0 + threadIdx.x;
      uint64_t v = 0ull;
      if (i < m) {
        int lo = 0, hi = nt - 1;  // last tile whose offset is <= i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (toff[mid] <= i) lo = mid; else hi = mid - 1;
        }
        v = crow[(int64_t)(t0 + lo) * kTopbKeys + (i - toff[lo])];
      }
      if (!in_lds) __syncthreads();
      if (i < m) dst[base + i] = v;
      if (!in_lds) __syncthreads();
    }
    base += m;
    __syncthreads();
  }
  uint64_t prefix = 0ull, mask = 0ull;  // n == need: every candidate is chosen
  if (need < (int)n)
    radix_select<true, 256>([&](int i) { return dst[i]; }, (int)n, need, rs, prefix, mask);
  auto index_of = [](uint64_t c) { return kRaw ? cand_index(c) : exact_key_index_desc(c); };

  // Chosen candidates per tile, counted in LDS (this workgroup owns every
  // tile of its problem) and stored once per tile. Blocks of kTileBlock
  // tiles bound the LDS for any history length.
  constexpr int kTileBlock = 1024;
  __shared__ uint32_t tcnt[kTileBlock];
  uint32_t* ch = a.chcount + (int64_t)h * a.NKT + kt_off[s];
  const int64_t bit0 = (int64_t)h * a.TL + h_off;
  for (int t0 = 0; t0 < ntile; t0 += kTileBlock) {
    const int nt = min(kTileBlock, ntile - t0);
    for (int i = threadIdx.x; i < nt; i += 256) tcnt[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < (int)n; i += 256) {
      const uint64_t c = dst[i];
      if (radix_taken<true>(c, prefix, mask)) {
        const int key = index_of(c);
        const int tl = key / kTopbKeys - t0;
        if (tl >= 0 && tl < nt) {
          atomicAdd(&tcnt[tl], 1u);
          const int64_t bit = bit0 + key;
          atomicOr(&a.bits[bit >> 5], 1u << (uint32_t)(bit & 31));
        }
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nt; i += 256) ch[t0 + i] = tcnt[i];
    __syncthreads();
  }
}

template <bool kRaw>
__global__ __launch_bounds__(256) void topb_write_kernel(const TopbArgs a, int32_t* __restrict__ sel_idx) {
  __shared__ RadixScratch<256> rs;
  const int tile = blockIdx.x, h = blockIdx.y;
  const int32_t* kt_off = a.plan + 2 * (a.S + 1);
  const int s = upper_seq(kt_off, a.S, tile);
  const int lt = tile - kt_off[s];
  const int h_off = a.cu_hist[s];
  const int L = a.cu_hist[s + 1] - h_off;
  const int prob = s * a.Hkv + h;
  const Threshold t = a.thr[prob];
  // the tile's scores are requested before the count of the tiles before it
  const float* srow = a.scores + (int64_t)h * a.TL + h_off;
  constexpr int PER = kTopbKeys / 256;
  const int k0 = lt * kTopbKeys + threadIdx.x * PER;
  float scv[PER];  // unconditional loads, clamped into the sequence (L >= 1 here)
#pragma unroll
  for (int e = 0; e < PER; ++e) scv[e] = srow[min(k0 + e, L - 1)];
  // this thread's PER keys span at most two bitmap words (PER divides 32)
  const int64_t bit = (int64_t)h * a.TL + h_off + k0;
  const uint64_t word2 = ((uint64_t)a.bits[(bit >> 5) + 1] << 32) | a.bits[bit >> 5];
  const uint32_t mine = (uint32_t)(word2 >> (bit & 31));

  uint32_t before = 0;
  for (int i = kt_off[s] + threadIdx.x; i < tile; i += 256)
    before += a.gtcount[(int64_t)h * a.NKT + i] + a.chcount[(int64_t)h * a.NKT + i];
  before = block_sum<256>(before, rs);

  uint32_t flags = 0, cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int key = k0 + e;
    if (key < L) {
      bool above, cand;
      if constexpr (kRaw) {
        const int bin = bin_of<true>(scv[e]);
        above = bin > t.bstar;
        cand = bin == t.bstar;
      } else {
        const double v = (double)scv[e];
        above = v > t.hi;
        cand = v >= t.lo;
      }
      const bool sel = t.bstar < 0 || above || (cand && (mine >> e & 1u));
      flags |= (uint32_t)sel << e;
      cnt += sel;
    }
  }
  uint32_t pos = before + block_exclusive_scan<256>(cnt, rs);
  int32_t* out = sel_idx + (int64_t)prob * a.kv_budget;
  const uint32_t b_eff = (uint32_t)min(a.kv_budget, L);
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if ((flags & (1u << e)) && pos < b_eff) out[pos++] = k0 + e;
}

hipError_t launch_topb(const Problem& p, const void* q, const void* k_hist, const int32_t* qidx,
                       char* ws, const Workspace& w, const float* scores, int32_t* sel_idx,
                       hipStream_t st) {
  if (p.NKT == 0) return hipSuccess;
  const bool raw = p.mode() == kModeDot;
  const ScoreBounds eb = score_bounds(p);
  TopbArgs a;
  a.cu_chunk = p.cu_chunk;
  a.cu_hist = p.cu_hist;
  a.plan = (const int32_t*)(ws + w.plan);
  a.S = p.S;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.TL = p.TL;
  a.NKT = p.NKT;
  a.kv_budget = p.kv_budget;
  a.eps = eb.eps;
  a.scores = scores;
  a.hist = (const uint32_t*)(ws + w.hist);
  a.thr = (Threshold*)(ws + w.thr);
  a.cand = (uint64_t*)(ws + w.cand);
  a.ctcount = (uint32_t*)(ws + w.ctcount);
  a.gtcount = (uint32_t*)(ws + w.gtcount);
  a.chcount = (uint32_t*)(ws + w.chcount);
  a.bits = (uint32_t*)(ws + w.bits);
  a.eps_row = eb.eps_row;
  a.q = q;
  a.k_hist = k_hist;
  a.qidx = qidx;
  a.q_budget = p.q_budget;
  a.nq_pad = p.nq_pad;
  a.variant = p.variant;
  a.row0 = (const double*)(ws + w.row0);
  a.gsel = ws + w.gsel;
  const dim3 grid((unsigned)p.NKT, (unsigned)p.Hkv);
  const dim3 cgrid((unsigned)(p.S * p.Hkv));
  if (raw) {
    hipLaunchKernelGGL((topb_filter_kernel<bf16, 128, true>), grid, dim3(256), 0, st, a);
  } else if (p.dtype == QUOKA_BF16) {
    if (p.D == 128) hipLaunchKernelGGL((topb_filter_kernel<bf16, 128, false>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((topb_filter_kernel<bf16, 64, false>), grid, dim3(256), 0, st, a);
  } else {
    if (p.D == 128) hipLaunchKernelGGL((topb_filter_kernel<float, 128, false>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((topb_filter_kernel<float, 64, false>), grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (raw) {
    hipLaunchKernelGGL(topb_cands_kernel<true>, cgrid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(topb_write_kernel<true>, grid, dim3(256), 0, st, a, sel_idx);
  } else {
    hipLaunchKernelGGL(topb_cands_kernel<false>, cgrid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(topb_write_kernel<false>, grid, dim3(256), 0, st, a, sel_idx);
  }
  return hipGetLastError();
}

}  // namespace quoka
