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

// ---- lane exchanges and wave reductions -------------------------------------
// Exchanges stay in registers: DPP moves inside each 16-lane row, then
// v_permlane16_swap / v_permlane32_swap across rows (a __shfl_xor would be an
// LDS round trip per step). In every reduction each step combines a lane's
// value with its partner's, so all lanes end with the same bits.
constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2): lane ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1): lane ^ 2
constexpr int kDppHalfMirror = 0x141; // lane 7 - i within each 8 (pairs the two quads)
constexpr int kDppMirror = 0x140;     // lane 15 - i within each 16 (pairs the two halves)

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}
template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<kCtrl>((uint32_t)v), hi = dpp_u32<kCtrl>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double v) {
  return __longlong_as_double((long long)dpp_u64<kCtrl>((uint64_t)__double_as_longlong(v)));
}
// The lane's value and its partner's (lane ^ 16, resp. lane ^ 32), as a pair
// whose order is the same in both lanes.
__device__ __forceinline__ void swap16(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}

// Sum / max over each 16-lane row (lanes 16r .. 16r + 15).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ uint32_t row16_sum(uint32_t v) {
  v += dpp_u32<kDppXor1>(v);
  v += dpp_u32<kDppXor2>(v);
  v += dpp_u32<kDppHalfMirror>(v);
  v += dpp_u32<kDppMirror>(v);
  return v;
}
// Sum over each aligned group of four lanes (the same bits in all four).
__device__ __forceinline__ double quad_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  return v;
}

// Sum over each aligned group of eight lanes.
__device__ __forceinline__ double oct_sum(double v) {
  v = quad_sum(v);
  v += dpp_f64<kDppHalfMirror>(v);
  return v;
}

// Sum of a double with its partner lane l ^ 16 (resp. l ^ 32), the same bits
// in both lanes.
__device__ __forceinline__ double pair16_sum(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t a0, b0, a1, b1;
  swap16((uint32_t)u, a0, b0);
  swap16((uint32_t)(u >> 32), a1, b1);
  return __longlong_as_double((long long)(((uint64_t)a1 << 32) | a0)) +
         __longlong_as_double((long long)(((uint64_t)b1 << 32) | b0));
}
__device__ __forceinline__ double pair32_sum(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t a0, b0, a1, b1;
  swap32((uint32_t)u, a0, b0);
  swap32((uint32_t)(u >> 32), a1, b1);
  return __longlong_as_double((long long)(((uint64_t)a1 << 32) | a0)) +
         __longlong_as_double((long long)(((uint64_t)b1 << 32) | b0));
}

// Sum / max of the four lanes l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float rows_sum(float v) {
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = __uint_as_float(a) + __uint_as_float(b);
  swap32(__float_as_uint(v), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float rows_max(float v) {
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = fmaxf(__uint_as_float(a), __uint_as_float(b));
  swap32(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ double rows_sum(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  uint32_t a0, b0, a1, b1;
  swap16((uint32_t)u, a0, b0);
  swap16((uint32_t)(u >> 32), a1, b1);
  v = __longlong_as_double((long long)(((uint64_t)a1 << 32) | a0)) +
      __longlong_as_double((long long)(((uint64_t)b1 << 32) | b0));
  const uint64_t w = (uint64_t)__double_as_longlong(v);
  swap32((uint32_t)w, a0, b0);
  swap32((uint32_t)(w >> 32), a1, b1);
  return __longlong_as_double((long long)(((uint64_t)a1 << 32) | a0)) +
         __longlong_as_double((long long)(((uint64_t)b1 << 32) | b0));
}
__device__ __forceinline__ uint32_t rows_sum(uint32_t v) {
  uint32_t a, b;
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

// Inclusive prefix sum over the 64 lanes: shifted adds inside each row
// (row_shr 1, 2, 4, 8, lanes shifted in from outside the row add zero), then
// lane 15 of each row into the next row and lane 31 into rows 2 and 3.
template <int kCtrl, int kRowMask, bool kBoundZero>
__device__ __forceinline__ uint32_t dpp_upd_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, kBoundZero);
}
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += dpp_upd_u32<0x111, 0xF, true>(x);   // row_shr:1
  x += dpp_upd_u32<0x112, 0xF, true>(x);   // row_shr:2
  x += dpp_upd_u32<0x114, 0xF, true>(x);   // row_shr:4
  x += dpp_upd_u32<0x118, 0xF, true>(x);   // row_shr:8
  x += dpp_upd_u32<0x142, 0xA, false>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_upd_u32<0x143, 0xC, false>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ uint32_t row16_min(uint32_t v) {
  v = min(v, dpp_u32<kDppXor1>(v));
  v = min(v, dpp_u32<kDppXor2>(v));
  v = min(v, dpp_u32<kDppHalfMirror>(v));
  v = min(v, dpp_u32<kDppMirror>(v));
  return v;
}
__device__ __forceinline__ uint32_t rows_min(uint32_t v) {
  uint32_t a, b;
  swap16(v, a, b);
  v = min(a, b);
  swap32(v, a, b);
  return min(a, b);
}

// ---- wave reductions (64 lanes, result in every lane) --------------------
__device__ __forceinline__ uint32_t wave_min(uint32_t v) { return rows_min(row16_min(v)); }
__device__ __forceinline__ float wave_sum(float v) { return rows_sum(row16_sum(v)); }
__device__ __forceinline__ double wave_sum(double v) { return rows_sum(row16_sum(v)); }
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return rows_sum(row16_sum(v)); }

// ---- order-preserving keys -------------------------------------------------
// Monotone map float -> uint32: a < b (as floats) <=> key(a) < key(b); -0 and
// +0 map to the same key. NaN is outside the contract.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_order_key (the key of -0 decodes to +0).
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The same monotone map for doubles: a < b <=> key(a) < key(b), -0 == +0.
__device__ __forceinline__ uint64_t double_order_key(double x) {
  if (x == 0.0) x = 0.0;
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double double_from_order_key(uint64_t k) {
  return __longlong_as_double((long long)((k & 0x8000000000000000ull) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k));
}

// Keys of the exact (fp64) re-evaluation near a selection boundary. Indices
// below 2^24 (the host rejects longer sequences); the value keeps the top
// bits of its double order key: 40 for history keys (sign, exponent and 28
// mantissa bits: two values closer than 2^-28 relative share a key and the
// lower index wins), 38 behind a two-bit class for chunk tokens.
constexpr int kExactIdxBits = 24;
constexpr uint32_t kExactIdxMask = (1u << kExactIdxBits) - 1u;
// larger is better: value desc, then index asc
__device__ __forceinline__ uint64_t exact_key_desc(double v, int idx) {
  return ((double_order_key(v) >> kExactIdxBits) << kExactIdxBits) |
         (uint64_t)(kExactIdxMask - (uint32_t)idx);
}
__device__ __forceinline__ int exact_key_index_desc(uint64_t k) {
  return (int)(kExactIdxMask - (uint32_t)(k & kExactIdxMask));
}
// smaller is better: class (0 sure in, 1 decided by value, 2 sure out), then
// value asc, then index asc
__device__ __forceinline__ uint64_t class_key_asc(uint32_t cls, double v, int idx) {
  const uint64_t val = cls == 1u ? (double_order_key(v) >> (64 - 38)) : 0ull;
  return ((uint64_t)cls << 62) | (val << kExactIdxBits) | (uint64_t)(uint32_t)idx;
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

// Eight consecutive row elements in their storage type, read as fp64 (bf16
// and fp32 convert exactly).
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ double operator[](int e) const { return (double)(float)v[e]; }
};
template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const float4*)p;
    b = *(const float4*)(p + 4);
  }
  __device__ __forceinline__ double operator[](int e) const {
    return e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : e == 3 ? a.w
         : e == 4 ? b.x : e == 5 ? b.y : e == 6 ? b.z : b.w;
  }
};

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
