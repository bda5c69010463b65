// K5: index-driven copy of the kept history rows into contiguous tiles.
// Source: "QUOKA Explained", "From scores to a smaller KV set" (when a key
// position is kept, its value comes along).
//   k_sel[s, h, b, :] = k_hist[cu_hist[s] + sel_idx[s, h, b], h, :]  (same for V)
// Rows whose index is -1 (or outside [0, L_s)) are written as zeros.
#include "common.h"
#include "internal.h"

namespace quoka {

// Each thread moves one 16-byte chunk of a K row and the same chunk of the V
// row; a workgroup covers 256 / (row bytes / 16) rows of one (sequence, head).
__global__ __launch_bounds__(256) void gather_kernel(
    const uint4* __restrict__ k_hist, const uint4* __restrict__ v_hist,
    const int32_t* __restrict__ cu_hist, const int32_t* __restrict__ sel_idx, int Hkv,
    int kv_budget, int chunks_per_row, uint4* __restrict__ k_sel, uint4* __restrict__ v_sel) {
  const int rows_per_block = 256 / chunks_per_row;
  const int s = blockIdx.z, h = blockIdx.y;
  const int b = blockIdx.x * rows_per_block + threadIdx.x / chunks_per_row;
  const int c = threadIdx.x % chunks_per_row;
  if (b >= kv_budget) return;
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int64_t prob = (int64_t)s * Hkv + h;
  const int idx = sel_idx[prob * kv_budget + b];
  const int64_t dst = (prob * kv_budget + b) * chunks_per_row + c;
  if (idx < 0 || idx >= L) {
    k_sel[dst] = make_uint4(0u, 0u, 0u, 0u);
    v_sel[dst] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int64_t src = ((int64_t)(h_off + idx) * Hkv + h) * chunks_per_row + c;
  const uint4 kv = k_hist[src];
  const uint4 vv = v_hist[src];
  k_sel[dst] = kv;
  v_sel[dst] = vv;
}

hipError_t launch_gather(const Problem& p, const void* k_hist, const void* v_hist,
                         const int32_t* sel_idx, void* k_sel, void* v_sel, hipStream_t st) {
  const int elem = p.dtype == QUOKA_BF16 ? 2 : 4;
  const int cpr = p.D * elem / 16;
  const int rpb = 256 / cpr;
  dim3 grid((unsigned)((p.kv_budget + rpb - 1) / rpb), (unsigned)p.Hkv, (unsigned)p.S);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, st, (const uint4*)k_hist,
                     (const uint4*)v_hist, p.cu_hist, sel_idx, p.Hkv, p.kv_budget, cpr,
                     (uint4*)k_sel, (uint4*)v_sel);
  return hipGetLastError();
}

}  // namespace quoka
