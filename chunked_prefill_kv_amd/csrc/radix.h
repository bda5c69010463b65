// Block-wide scans and an exact radix select over unique 64-bit keys, for
// workgroups of NT threads (NT = 256 or 1024).
#pragma once

#include "common.h"

namespace quoka {

template <int NT>
struct RadixScratch {
  static constexpr int W = NT / 64;
  alignas(16) uint32_t hist[2][256];  // digit histograms, alternating between passes
  uint32_t wsum[W];
  uint64_t wand[W], wor[W];
  uint32_t digit;
  uint32_t rem;
  uint32_t done;
};

// Inclusive prefix sum of one value per thread over the block.
template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, RadixScratch<NT>& rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) rs.wsum[w] = x;
  __syncthreads();
  uint32_t add = 0;
  for (int i = 0; i < w; ++i) add += rs.wsum[i];
  __syncthreads();
  return x + add;
}

template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, RadixScratch<NT>& rs) {
  return block_inclusive_scan<NT>(v, rs) - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, RadixScratch<NT>& rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_sum(v);
  if (lane == 0) rs.wsum[w] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t += rs.wsum[i];
  __syncthreads();
  return t;
}

// Minimum / maximum of one value per thread over the block.
template <int NT>
__device__ __forceinline__ uint32_t block_min(uint32_t v, RadixScratch<NT>& rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_min(v);
  if (lane == 0) rs.wsum[w] = v;
  __syncthreads();
  uint32_t t = ~0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) t = min(t, rs.wsum[i]);
  __syncthreads();
  return t;
}
template <int NT>
__device__ __forceinline__ uint32_t block_max(uint32_t v, RadixScratch<NT>& rs) {
  return ~block_min<NT>(~v, rs);
}

// Exact selection of the k smallest (kLargest = false) or k largest
// (kLargest = true) of N unique 64-bit keys key_of(0..N-1), 1 <= k < N.
// Result: the selected keys are exactly those with
//     (key & mask) <= prefix   (smallest)   or   (key & mask) >= prefix (largest).
// The bits all keys share are skipped first; then 8-bit digits are resolved
// from the top, histogramming the keys that still match, until the bucket at
// the boundary is taken whole (or every digit is fixed, when prefix is the
// k-th key itself).
// Bitwise and / or of a and o over the wave (result in every lane).
__device__ __forceinline__ void wave_and_or(uint64_t& a, uint64_t& o) {
  a &= dpp_u64<kDppXor1>(a); o |= dpp_u64<kDppXor1>(o);
  a &= dpp_u64<kDppXor2>(a); o |= dpp_u64<kDppXor2>(o);
  a &= dpp_u64<kDppHalfMirror>(a); o |= dpp_u64<kDppHalfMirror>(o);
  a &= dpp_u64<kDppMirror>(a); o |= dpp_u64<kDppMirror>(o);
  uint32_t x0, y0, x1, y1;
  swap16((uint32_t)a, x0, y0); swap16((uint32_t)(a >> 32), x1, y1);
  a = (((uint64_t)x1 << 32) | x0) & (((uint64_t)y1 << 32) | y0);
  swap32((uint32_t)a, x0, y0); swap32((uint32_t)(a >> 32), x1, y1);
  a = (((uint64_t)x1 << 32) | x0) & (((uint64_t)y1 << 32) | y0);
  swap16((uint32_t)o, x0, y0); swap16((uint32_t)(o >> 32), x1, y1);
  o = (((uint64_t)x1 << 32) | x0) | (((uint64_t)y1 << 32) | y0);
  swap32((uint32_t)o, x0, y0); swap32((uint32_t)(o >> 32), x1, y1);
  o = (((uint64_t)x1 << 32) | x0) | (((uint64_t)y1 << 32) | y0);
}

template <bool kLargest, int NT, typename KeyFn>
__device__ void radix_select(KeyFn key_of, int N, int k, RadixScratch<NT>& rs, uint64_t& prefix,
                             uint64_t& mask) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint64_t a = ~0ull, o = 0ull;
  for (int i = threadIdx.x; i < N; i += NT) {
    const uint64_t key = key_of(i);
    a &= key;
    o |= key;
  }
  wave_and_or(a, o);
  if (lane == 0) { rs.wand[w] = a; rs.wor[w] = o; }
  __syncthreads();
  a = ~0ull;
  o = 0ull;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) { a &= rs.wand[i]; o |= rs.wor[i]; }
  __syncthreads();
  const uint64_t diff = a ^ o;
  if (diff == 0ull) {  // a single distinct key
    prefix = a;
    mask = ~0ull;
    return;
  }
  const int top = 63 - __clzll(diff);
  const int shift0 = (top / 8) * 8;
  mask = shift0 + 8 >= 64 ? 0ull : (~0ull << (shift0 + 8));
  prefix = a & mask;
  uint32_t rem = (uint32_t)k;
  // Each digit pass: one histogram of the keys still matching, then a single
  // wave scans its 256 bins (4 per lane) and picks the digit. The two
  // histograms alternate, so the one for the next pass is cleared by that
  // wave meanwhile: two barriers per pass.
  for (int i = threadIdx.x; i < 512; i += NT) (&rs.hist[0][0])[i] = 0u;
  __syncthreads();
  int hb = 0;
  for (int shift = shift0; shift >= 0; shift -= 8, hb ^= 1) {
    uint32_t* hist = rs.hist[hb];
    for (int i = threadIdx.x; i < N; i += NT) {
      const uint64_t key = key_of(i);
      if ((key & mask) == prefix) {
        uint32_t d = (uint32_t)(key >> shift) & 255u;
        if (kLargest) d = 255u - d;
        atomicAdd(&hist[d], 1u);
      }
    }
    __syncthreads();
    if (w == 0) {
      const uint4 c4 = ((const uint4*)hist)[lane];
      const uint32_t tot = c4.x + c4.y + c4.z + c4.w;
      uint32_t excl = wave_inclusive_scan(tot) - tot;  // keys in bins below 4 * lane
      const uint32_t c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c[e] > 0 && excl < rem && rem <= excl + c[e]) {
          rs.digit = 4 * lane + e;
          rs.rem = rem - excl;
          rs.done = excl + c[e] == rem;
        }
        excl += c[e];
      }
      ((uint4*)rs.hist[hb ^ 1])[lane] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    uint32_t d = rs.digit;
    rem = rs.rem;
    const bool done = rs.done != 0u;
    if (kLargest) d = 255u - d;
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    if (done) break;
  }
}

template <bool kLargest>
__device__ __forceinline__ bool radix_taken(uint64_t key, uint64_t prefix, uint64_t mask) {
  return kLargest ? (key & mask) >= prefix : (key & mask) <= prefix;
}

// Top-B threshold bin from a complete score histogram (kScoreBins linear bins
// over [-1, 1]): bin b* holding the B_eff-th largest score, the number of
// keys above it, and how many of b*'s keys are still needed. Block of NT
// threads; every thread returns the same values.
template <int NT>
__device__ void find_threshold_bin(const uint32_t* __restrict__ h, int L, int B_eff,
                                   RadixScratch<NT>& rs, int* bstar, int* above, int* need) {
  __shared__ int sh[3];
  if (B_eff >= L) {
    *bstar = -1; *above = L; *need = 0;
    return;
  }
  // thread i owns PER bins counting down from the top
  constexpr int PER = kScoreBins / NT;
  uint32_t c[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    c[e] = h[kScoreBins - 1 - (threadIdx.x * PER + e)];
    tot += c[e];
  }
  uint32_t cum = block_exclusive_scan<NT>(tot, rs);  // keys in higher bins
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

}  // namespace quoka
