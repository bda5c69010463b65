// Block-wide scans and an exact radix select over unique 64-bit keys, for
// 256-thread workgroups.
#pragma once

#include "common.h"

namespace quoka {

struct RadixScratch {
  uint32_t hist[256];
  uint32_t wsum[4];
  uint32_t digit;
  uint32_t rem;
};

// Inclusive prefix sum of one value per thread over a 256-thread block.
__device__ __forceinline__ uint32_t block_inclusive_scan_256(uint32_t v, RadixScratch& rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) rs.wsum[w] = x;
  __syncthreads();
  uint32_t add = 0;
  for (int i = 0; i < w; ++i) add += rs.wsum[i];
  __syncthreads();
  return x + add;
}

__device__ __forceinline__ uint32_t block_exclusive_scan_256(uint32_t v, RadixScratch& rs) {
  return block_inclusive_scan_256(v, rs) - v;
}

__device__ __forceinline__ uint32_t block_sum_256(uint32_t v, RadixScratch& rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) rs.wsum[w] = v;
  __syncthreads();
  const uint32_t t = rs.wsum[0] + rs.wsum[1] + rs.wsum[2] + rs.wsum[3];
  __syncthreads();
  return t;
}

// The k-th smallest (kLargest = false) or k-th largest (kLargest = true) of N
// unique 64-bit keys key_of(0..N-1), 1 <= k <= N. Eight passes of 8-bit
// digits from the top; each pass histograms the keys that still match the
// digits fixed so far. Exact: the result is a key that occurs in the input.
template <bool kLargest, typename KeyFn>
__device__ uint64_t radix_select_kth(KeyFn key_of, int N, int k, RadixScratch& rs) {
  uint64_t prefix = 0, mask = 0;
  uint32_t rem = (uint32_t)k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    rs.hist[threadIdx.x] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += 256) {
      const uint64_t key = key_of(i);
      if ((key & mask) == prefix) {
        uint32_t d = (uint32_t)(key >> shift) & 255u;
        if (kLargest) d = 255u - d;
        atomicAdd(&rs.hist[d], 1u);
      }
    }
    __syncthreads();
    const uint32_t v = rs.hist[threadIdx.x];
    const uint32_t incl = block_inclusive_scan_256(v, rs);
    const uint32_t excl = incl - v;
    if (v > 0 && excl < rem && rem <= incl) {
      rs.digit = threadIdx.x;
      rs.rem = rem - excl;
    }
    __syncthreads();
    uint32_t d = rs.digit;
    rem = rs.rem;
    if (kLargest) d = 255u - d;
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    __syncthreads();
  }
  return prefix;
}

}  // namespace quoka
