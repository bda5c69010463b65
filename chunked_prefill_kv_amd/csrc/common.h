// Device helpers shared by the QUOKA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace quoka {

constexpr int kWave = 64;

// ---- element conversion --------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// ---- wave reductions (64 lanes, result in every lane) --------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---- order-preserving keys -------------------------------------------------
// Monotone map float -> uint32: a < b (as floats) <=> key(a) < key(b); -0 and
// +0 map to the same key. NaN is outside the contract.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Linear histogram bin of a score in [-1, 1] (cosine-derived scores are
// bounded). Monotone non-decreasing in s; out-of-range values clamp.
constexpr int kScoreBins = 2048;
__device__ __forceinline__ int score_bin(float s) {
  float x = (s + 1.0f) * (0.5f * kScoreBins);
  x = fminf(fmaxf(x, 0.0f), (float)(kScoreBins - 1));
  return (int)x;
}

// Histogram bin of an unbounded score (raw dot products): the top 11 bits of
// its order key. Monotone non-decreasing over all floats; coarse (4 bins per
// binade), which only makes the top-B refinement see more candidates.
__device__ __forceinline__ int score_bin_raw(float s) { return (int)(float_order_key(s) >> 21); }
static_assert(kScoreBins == 2048, "score_bin_raw yields 11 bits");

// ---- buffer loads ----------------------------------------------------------
// Raw buffer resource over [p, p + nbytes): loads at byte offsets >= nbytes
// return zeros (bounds checked in hardware on the VGPR offset). p and nbytes
// must be the same in every lane of the wave; they are moved to scalar
// registers explicitly (values the compiler computed in VGPRs, such as
// integer quotients, would otherwise be legalised with a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t nbytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* pu = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, (int)__builtin_amdgcn_readfirstlane(nbytes),
                                           0x00020000);
}
__device__ __forceinline__ bf16x8 buffer_load_bf16x8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return __builtin_bit_cast(bf16x8, v);
}

// ---- block-wide copies ------------------------------------------------------
// dst[i] = src[i] for i < n by a block of NT threads, with up to U loads per
// thread in flight before their stores (a plain strided loop waits for each
// load in turn).
template <int NT, int U, typename T>
__device__ __forceinline__ void block_copy(T* __restrict__ dst, const T* __restrict__ src, int n) {
  for (int base = 0; base < n; base += NT * U) {
    T v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      if (i < n) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NT + (int)threadIdx.x;
      if (i < n) dst[i] = v[u];
    }
  }
}

// Largest s in [0, n) with off[s] <= v, for non-decreasing off[0..n].
__device__ __forceinline__ int upper_seq(const int32_t* off, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace quoka
