// Probes that confirm, on the chip at hand, the peaks the rooflines divide by:
// the dense bf16 MFMA rate, the HBM streaming rates and the shader clock.
// Built into its own library (libquoka_peaks.so); only the bench loads it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef __bf16 pk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pk_f32x16 __attribute__((ext_vector_type(16)));

// Four independent accumulation chains of v_mfma_f32_32x32x16_bf16 per wave
// (32768 flop each), so that issue, not the chain latency, bounds the rate.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* __restrict__ out) {
  pk_bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((float)((threadIdx.x + e) & 7) * 0.125f);
    b[e] = (__bf16)((float)((threadIdx.x * 3 + e) & 7) * 0.0625f);
  }
  pk_f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) sum += c0[e] + c1[e] + c2[e] + c3[e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

// Streaming read of n float4 (16-byte loads, grid-stride, eight in flight).
__global__ __launch_bounds__(256) void peak_read_kernel(const float4* __restrict__ p, size_t n,
                                                         float* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  float acc = 0.f;
  for (; i + 7 * stride < n; i += 8 * stride) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u].x + v[u].w;
  }
  for (; i < n; i += stride) acc += p[i].x;
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// The shader cycle counter against the 100 MHz real-time counter over a
// dependent arithmetic loop of one wave.
__global__ __launch_bounds__(64) void peak_clock_kernel(int iters,
                                                        unsigned long long* __restrict__ out,
                                                        float* __restrict__ sink) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  float x = (float)threadIdx.x;
  for (int i = 0; i < iters; ++i) x = fmaf(x, 0.999999f, 0.5f);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[threadIdx.x] = x;
  if (threadIdx.x == 0) {
    out[0] = t0;
    out[1] = t1;
    out[2] = r0;
    out[3] = r1;
  }
}

extern "C" {

// blocks x 256 threads, `iters` rounds of four MFMAs per wave; out holds
// blocks * 256 floats. Returns a hipError_t.
int quoka_peaks_mfma(int blocks, int iters, float* out, hipStream_t st) {
  if (blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, st, iters, out);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from buf with blocks x 256 threads; out
// holds blocks * 256 floats.
int quoka_peaks_read(const void* buf, size_t bytes, int blocks, float* out, hipStream_t st) {
  if (!buf || !out || blocks < 1 || bytes % 16) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const float4*)buf, bytes / 16, out);
  return (int)hipGetLastError();
}

// out[0..3] = shader counter before / after, real-time counter before / after;
// sink holds 64 floats.
int quoka_peaks_clock(int iters, unsigned long long* out, float* sink, hipStream_t st) {
  if (iters < 1 || !out || !sink) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(peak_clock_kernel, dim3(1), dim3(64), 0, st, iters, out, sink);
  return (int)hipGetLastError();
}

// What the runtime reports: peak clock (kHz), memory clock (kHz), bus width
// (bits) and compute units of the current device.
int quoka_peaks_device(int* clock_khz, int* mem_clock_khz, int* bus_bits, int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(bus_bits, hipDeviceAttributeMemoryBusWidth, dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  return (int)e;
}

}  // extern "C"
