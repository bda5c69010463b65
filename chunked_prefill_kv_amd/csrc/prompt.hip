// Whole-prompt chunked prefill of one sequence: the per-chunk offsets the
// chunk-by-chunk loop passes to the per-chunk path, written on the device so
// that the loop copies nothing from the host.
// Sources: QUOKA paper summary (hw-hk.tistory.com/367), "Background >
// Chunked prefill" (chunk i covers tokens [i B_cp, min(T, (i+1) B_cp)) and
// its history is every earlier token).
#include "common.h"
#include "internal.h"

namespace quoka {

// cu[4 i .. 4 i + 3] = {0, C_i, 0, L_i}: the cu_chunk and cu_hist arrays of
// chunk i as a one-sequence problem.
__global__ __launch_bounds__(256) void prompt_offsets_kernel(int T, int chunk_len, int nch,
                                                             int32_t* __restrict__ cu) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < nch; i += gridDim.x * 256) {
    const int a = i * chunk_len, b = min(T, a + chunk_len);
    cu[4 * i + 0] = 0;
    cu[4 * i + 1] = b - a;
    cu[4 * i + 2] = 0;
    cu[4 * i + 3] = a;
  }
}

hipError_t launch_prompt_offsets(int T, int chunk_len, int nch, int32_t* cu, hipStream_t st) {
  const int grid = (nch + 255) / 256;
  hipLaunchKernelGGL(prompt_offsets_kernel, dim3(grid), dim3(256), 0, st, T, chunk_len, nch, cu);
  return hipGetLastError();
}

}  // namespace quoka
