// Checks of the QUOKA_DEBUG mode and of quoka_check_selection.
//
// The kernels read the arguments' bytes and record, per check, the smallest
// flat index that breaks it (atomicMin into a small per-device array); the
// host copies the array back, synchronises the stream and turns the first
// failure into a status and a message. Nothing here writes an argument.
//
// What is checked is what the entry points state as their preconditions and
// what the selection promises its callers ("QUOKA Explained", "From scores to
// a smaller KV set": the kept set is B keys of the history; the selection
// writes them ascending, padded with -1):
//   - the device offset arrays hold the host copies' values;
//   - every Q/K/V element a kernel reads is finite (no Inf / NaN bit pattern);
//   - kept-index inputs are -1 or a position of the sequence's history;
//   - kept-index outputs of (s, h) are strictly ascending positions in
//     [0, L_s) for b < B_eff and -1 from B_eff on.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "debug.h"
#include "internal.h"

namespace quoka {

namespace {

// per check: the smallest failing flat index, ULLONG_MAX when none failed
__device__ __align__(256) unsigned long long debug_first[kDebugSlots];

__global__ __launch_bounds__(64) void debug_clear_kernel(unsigned long long* first) {
  if (threadIdx.x < kDebugSlots) first[threadIdx.x] = ULLONG_MAX;
}

// An element is non-finite when its exponent bits are all set. A 32-bit
// word holds one fp32 value (exponent at bits 23..30) or two bf16 values
// (exponents at bits 7..14 and 23..30).
__device__ bool lo_bf16_bad(uint32_t v) { return (v & 0x7f80u) == 0x7f80u; }
__device__ bool hi_bad(uint32_t v) { return (v & 0x7f800000u) == 0x7f800000u; }

// nwords 32-bit words in rows of words_per_row (d is 64 or 128, so a row is
// whole words); records the flat element index of the first non-finite
// value. kDebugRowsSel skips the rows past B_eff, which no kernel reads.
__global__ __launch_bounds__(256) void debug_finite_kernel(
    const uint32_t* __restrict__ base, int64_t nwords, int words_per_row, int elems_per_word,
    bool bf, int mode, int Hkv, int kv_budget, const int32_t* __restrict__ cu_hist,
    unsigned long long* first, int slot) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) {
    if (mode == kDebugRowsSel) {
      // [S, Hkv, kv_budget, d]: only the first B_eff rows of (s, h) are read
      const int64_t row = i / words_per_row;
      const int b = (int)(row % kv_budget);
      const int s = (int)(row / kv_budget / Hkv);
      const int L = cu_hist[s + 1] - cu_hist[s];
      if (b >= min(kv_budget, L)) continue;
    }
    const uint32_t v = base[i];
    const bool lo = bf && lo_bf16_bad(v);
    if (lo || hi_bad(v))  // element 2i (low half) before 2i + 1
      atomicMin(&first[slot], (unsigned long long)i * elems_per_word + (bf && !lo ? 1 : 0));
  }
}

// kept indices [S, Hkv, kv_budget]: inputs (kDebugIdxInput) must be -1 or in
// [0, L_s); outputs (kDebugIdxSelection) must be ascending in [0, L_s) below
// B_eff and -1 from there on.
__global__ __launch_bounds__(256) void debug_index_kernel(
    const int32_t* __restrict__ sel, int64_t n, int Hkv, int kv_budget,
    const int32_t* __restrict__ cu_hist, int mode, unsigned long long* first, int slot) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int b = (int)(i % kv_budget);
    const int s = (int)(i / kv_budget / Hkv);
    const int L = cu_hist[s + 1] - cu_hist[s];
    const int v = sel[i];
    bool ok;
    if (mode == kDebugIdxInput) {
      ok = v == -1 || (v >= 0 && v < L);
    } else {
      const int B_eff = min(kv_budget, L);
      ok = b < B_eff ? (v >= 0 && v < L && (b == 0 || v > sel[i - 1])) : v == -1;
    }
    if (!ok) atomicMin(&first[slot], (unsigned long long)i);
  }
}

std::mutex g_debug_mu;

quoka_status debug_slots(unsigned long long** out) {
  static unsigned long long* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QUOKA_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(QUOKA_EUNSUPPORTED, "device ordinal %d", dev);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_first));
    if (e != hipSuccess || !ptr)
      return fail(QUOKA_EHIP, "hipGetSymbolAddress(debug_first): %s", hipGetErrorString(e));
    addr[dev] = (unsigned long long*)ptr;
  }
  *out = addr[dev];
  return QUOKA_OK;
}

unsigned grid_for(int64_t n) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 2048));
}

const char* tensor_name(int slot) {
  switch (slot) {
    case kDbgQ: return "q";
    case kDbgKHist: return "k_hist";
    case kDbgVHist: return "v_hist";
    case kDbgKChunk: return "k_chunk";
    case kDbgVChunk: return "v_chunk";
    case kDbgKSel: return "k_sel";
    case kDbgVSel: return "v_sel";
    case kDbgSelIn: return "sel_idx";
    case kDbgSelOut: return "sel_idx";
    case kDbgK: return "k";
    case kDbgV: return "v";
  }
  return "?";
}

}  // namespace

bool debug_mode() {
  const char* v = std::getenv("QUOKA_DEBUG");
  return v && v[0] && std::strcmp(v, "0") != 0;
}

quoka_status debug_offsets(const Problem& p) {
  std::vector<int32_t> dc(p.S + 1), dh(p.S + 1);
  hipError_t e = hipMemcpy(dc.data(), p.cu_chunk, (p.S + 1) * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess)
    e = hipMemcpy(dh.data(), p.cu_hist, (p.S + 1) * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess)
    return fail(QUOKA_EHIP, "QUOKA_DEBUG: reading the device offsets: %s", hipGetErrorString(e));
  for (int s = 0; s <= p.S; ++s) {
    if (dc[s] != p.cu_chunk_h[s])
      return fail(QUOKA_EINVAL, "QUOKA_DEBUG: cu_chunk[%d] is %d on the device, %d on the host",
                  s, dc[s], p.cu_chunk_h[s]);
    if (dh[s] != p.cu_hist_h[s])
      return fail(QUOKA_EINVAL, "QUOKA_DEBUG: cu_hist[%d] is %d on the device, %d on the host",
                  s, dh[s], p.cu_hist_h[s]);
  }
  return QUOKA_OK;
}

quoka_status debug_run(const Problem& p, const DebugItem* items, int n, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_debug_mu);
  unsigned long long* first = nullptr;
  quoka_status rc = debug_slots(&first);
  if (rc != QUOKA_OK) return rc;
  hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(64), 0, st, first);
  const bool bf = p.dtype == QUOKA_BF16;
  const int epw = bf ? 2 : 1;  // elements per 32-bit word
  for (int i = 0; i < n; ++i) {
    const DebugItem& it = items[i];
    if (!it.ptr || it.count == 0) continue;
    if (it.kind == kDebugIdxInput || it.kind == kDebugIdxSelection) {
      hipLaunchKernelGGL(debug_index_kernel, dim3(grid_for(it.count)), dim3(256), 0, st,
                         (const int32_t*)it.ptr, it.count, p.Hkv, p.kv_budget, p.cu_hist,
                         it.kind, first, it.slot);
    } else {
      const int64_t nwords = it.count / epw;  // count: elements; rows of d >= 64
      hipLaunchKernelGGL(debug_finite_kernel, dim3(grid_for(nwords)), dim3(256), 0, st,
                         (const uint32_t*)it.ptr, nwords, p.D / epw, epw, bf, it.kind, p.Hkv,
                         p.kv_budget, p.cu_hist, first, it.slot);
    }
  }
  unsigned long long host[kDebugSlots];
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(host, first, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(QUOKA_EHIP, "QUOKA_DEBUG checks: %s", hipGetErrorString(e));
  for (int i = 0; i < n; ++i) {
    const DebugItem& it = items[i];
    const unsigned long long f = host[it.slot];
    if (f == ULLONG_MAX) continue;
    const char* name = tensor_name(it.slot);
    if (it.kind == kDebugIdxInput || it.kind == kDebugIdxSelection) {
      const int64_t b = (int64_t)(f % p.kv_budget), h = (int64_t)(f / p.kv_budget % p.Hkv),
                    s = (int64_t)(f / p.kv_budget / p.Hkv);
      if (it.kind == kDebugIdxInput)
        return fail(QUOKA_EINVAL,
                    "QUOKA_DEBUG: %s[s=%lld, h=%lld, b=%lld] is neither -1 nor a position of "
                    "the sequence's history",
                    name, (long long)s, (long long)h, (long long)b);
      return fail(QUOKA_ECHECK,
                  "QUOKA_DEBUG: %s[s=%lld, h=%lld, b=%lld] breaks the kept-index layout "
                  "(ascending positions in [0, L_s) below B_eff, -1 after)",
                  name, (long long)s, (long long)h, (long long)b);
    }
    const long long row = (long long)(f / p.D), col = (long long)(f % p.D);
    return fail(QUOKA_EINVAL, "QUOKA_DEBUG: %s holds a non-finite value (row %lld, element %lld)",
                name, row, col);
  }
  return QUOKA_OK;
}

}  // namespace quoka
