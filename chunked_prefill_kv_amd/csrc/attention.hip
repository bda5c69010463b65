// K6: chunk attention over [kept history | own chunk] with a causal mask.
//   O[t, j] = softmax(q_{t,j} [K_sel ; K_chunk[0..t]]^T * scale) [V_sel ; V_chunk[0..t]]
// The kept history keys are visible to every chunk query; the chunk's own keys
// follow the causal mask with the diagonal included. The original query heads
// (not their group mean) attend.
// Sources: QUOKA paper summary (hw-hk.tistory.com/367), "Background > Chunked
// prefill" (chunk i attends to the previous chunks' K/V concatenated with its
// own under a mask that enforces causality inside the chunk) and "QUOKA
// Method" (the reduced KV set is fed to a dense attention kernel); "QUOKA
// Explained", "MEAN and MAX do different jobs" (the original query heads do
// the attention).
#include "common.h"
#include "internal.h"

namespace quoka {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// VALU path (fp32): one wave per 64 query tokens of one query head, one token
// per lane, K/V tiles of 32 rows staged in LDS and read by broadcast, online
// softmax per key.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k_sel, const T* __restrict__ v_sel,
    const T* __restrict__ k_chunk, const T* __restrict__ v_chunk,
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist, int Hq, int Hkv,
    int G, int kv_budget, float scale_log2, T* __restrict__ out) {
  constexpr int KT = 32;
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];
  const int s = blockIdx.z, j = blockIdx.y, h = j / G;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int t0 = blockIdx.x * 64;
  if (t0 >= C) return;
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, L);
  const int lane = threadIdx.x;
  const int t = t0 + lane;
  const bool valid = t < C;

  float qv[D], o[D];
  const T* qrow = q + ((int64_t)(c_off + (valid ? t : 0)) * Hq + j) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = to_f32(qrow[d]) * scale_log2;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int64_t prob = (int64_t)s * Hkv + h;
  const int t_end = min(C, t0 + 64);  // keys [0, t_end) of the chunk are needed

  for (int phase = 0; phase < 2; ++phase) {
    const int nkeys = phase == 0 ? B_eff : t_end;
    const T* kb = phase == 0 ? k_sel + prob * kv_budget * D : k_chunk + ((int64_t)c_off * Hkv + h) * D;
    const T* vb = phase == 0 ? v_sel + prob * kv_budget * D : v_chunk + ((int64_t)c_off * Hkv + h) * D;
    const int64_t stride = phase == 0 ? D : (int64_t)Hkv * D;
    for (int k0 = 0; k0 < nkeys; k0 += KT) {
      __syncthreads();
      for (int idx = lane; idx < KT * D; idx += 64) {
        const int r = idx / D, c = idx % D;
        const bool ok = k0 + r < nkeys;
        Ks[r][c] = ok ? to_f32(kb[(int64_t)(k0 + r) * stride + c]) : 0.f;
        Vs[r][c] = ok ? to_f32(vb[(int64_t)(k0 + r) * stride + c]) : 0.f;
      }
      __syncthreads();
      const int kn = min(KT, nkeys - k0);
      for (int kk = 0; kk < kn; ++kk) {
        if (phase == 1 && k0 + kk > t) break;
        float x = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) x = fmaf(qv[d], Ks[kk][d], x);
        const float m_new = fmaxf(m, x);
        const float corr = exp2f(m - m_new);
        const float p = exp2f(x - m_new);
        l = l * corr + p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(o[d], corr, p * Vs[kk][d]);
        m = m_new;
      }
    }
  }
  if (valid) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    T* orow = out + ((int64_t)(c_off + t) * Hq + j) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = from_f32<T>(o[d] * inv);
  }
}

// ---------------------------------------------------------------------------
// MFMA path (bf16): flash-style online softmax on v_mfma_f32_32x32x16_bf16.
// A workgroup of 4 waves owns 128 packed query rows of one (sequence, KV
// head); row r is token r / G, query head h*G + r % G, so the G heads that
// share the KV head share every K/V tile. Each wave owns 32 rows.
//   S^T = K Q^T  : A = K tile rows from LDS, B = the wave's Q held in VGPRs,
//                  C lane l = query column l%32, 16 key rows.
//   O^T += V^T P^T: A = V^T from LDS (stored transposed), B = P taken straight
//                  from the S^T accumulators; the 16 keys of a k-step are the
//                  ones the lane already holds, so P never leaves registers.
// K/V tiles of 64 keys: first the kept history (unmasked past B_eff), then
// the chunk's keys up to the workgroup's last token (causal mask per row).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_sel, const bf16* __restrict__ v_sel,
    const bf16* __restrict__ k_chunk, const bf16* __restrict__ v_chunk,
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist, int Hq, int Hkv,
    int G, int kv_budget, float scale_log2, bf16* __restrict__ out) {
  constexpr int KT = 64, NDS = D / 16, NDB = D / 32;
  constexpr int KSTR = D + 8;   // padded row strides (elements)
  constexpr int VSTR = KT + 4;
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * KSTR];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * VSTR];

  const int s = blockIdx.z, h = blockIdx.y;
  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int rows = C * G;
  const int ntile = (rows + 127) / 128;
  if ((int)blockIdx.x >= ntile) return;
  const int tile = ntile - 1 - (int)blockIdx.x;  // longest rows first
  const int h_off = cu_hist[s];
  const int L = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, L);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hi = lane >> 5;
  const int r = tile * 128 + wave * 32 + col;
  const bool rvalid = r < rows;
  const int t = rvalid ? r / G : 0;
  const int jh = h * G + (rvalid ? r % G : 0);

  bf16x8 qreg[NDS];
  {
    const bf16* qrow = q + ((int64_t)(c_off + t) * Hq + jh) * D + hi * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      bf16x8 v = *(const bf16x8*)(qrow + ds * 16);
      qreg[ds] = rvalid ? v : (bf16x8){};
    }
  }
  const int t_last = min(C - 1, (tile * 128 + 127) / G);
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, l_run = 0.f;

  const int64_t prob = (int64_t)s * Hkv + h;
  const bf16* k1 = k_sel + prob * kv_budget * D;
  const bf16* v1 = v_sel + prob * kv_budget * D;
  const bf16* k2 = k_chunk + ((int64_t)c_off * Hkv + h) * D;
  const bf16* v2 = v_chunk + ((int64_t)c_off * Hkv + h) * D;
  const int n1 = (B_eff + KT - 1) / KT;
  const int n2 = (t_last + KT) / KT;

  for (int it = 0; it < n1 + n2; ++it) {
    const bool ph1 = it < n1;
    const int kbase = (ph1 ? it : it - n1) * KT;
    const int klim = ph1 ? B_eff : t_last + 1;
    const bf16* kp = ph1 ? k1 : k2;
    const bf16* vp = ph1 ? v1 : v2;
    const int64_t rstride = ph1 ? (int64_t)D : (int64_t)Hkv * D;

    __syncthreads();
    for (int cc = threadIdx.x; cc < KT * D / 8; cc += 256) {
      const int kr = cc / (D / 8), part = cc % (D / 8);
      const int key = kbase + kr;
      bf16x8 kv = (bf16x8){}, vv = (bf16x8){};
      if (key < klim) {
        kv = *(const bf16x8*)(kp + key * rstride + part * 8);
        vv = *(const bf16x8*)(vp + key * rstride + part * 8);
      }
      *(bf16x8*)&Ks[kr * KSTR + part * 8] = kv;
#pragma unroll
      for (int e = 0; e < 8; ++e) Vt[(part * 8 + e) * VSTR + kr] = vv[e];
    }
    __syncthreads();

    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sacc[sb] = (f32x16){};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 a = *(const bf16x8*)&Ks[(sb * 32 + col) * KSTR + ds * 16 + hi * 8];
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], sacc[sb], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int key = kbase + sb * 32 + hi * 4 + jj + 8 * i;
          const bool ok = rvalid && (ph1 ? key < B_eff : key <= t);
          const float x = ok ? sacc[sb][i * 4 + jj] * scale_log2 : -INFINITY;
          sacc[sb][i * 4 + jj] = x;
          mx = fmaxf(mx, x);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - base);
    float ps = 0.f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p = exp2f(sacc[sb][i * 4 + jj] - base);
          ps += p;
          pb[sb][i >> 1][(i & 1) * 4 + jj] = (bf16)p;
        }
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16* vrow = &Vt[(db * 32 + col) * VSTR];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kb0 = sb * 32 + kk * 16 + hi * 4;
          const bf16x4 lo4 = *(const bf16x4*)(vrow + kb0);
          const bf16x4 hi4 = *(const bf16x4*)(vrow + kb0 + 8);
          const bf16x8 a = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[sb][kk], oacc[db], 0, 0, 0);
        }
    }
  }

  if (rvalid) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    bf16* orow = out + ((int64_t)(c_off + t) * Hq + jh) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 v;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = (bf16)(oacc[db][i * 4 + jj] * inv);
        *(bf16x4*)(orow + db * 32 + hi * 4 + 8 * i) = v;
      }
  }
}

hipError_t launch_attention(const Problem& p, const void* q, const void* k_sel,
                            const void* v_sel, const void* k_chunk, const void* v_chunk,
                            float scale, void* out, hipStream_t st) {
  if (p.maxC == 0) return hipSuccess;
  const float sl2 = scale * kLog2e;
  if (p.dtype == QUOKA_BF16) {
    const int ntile = (p.maxC * p.G + 127) / 128;
    dim3 grid((unsigned)ntile, (unsigned)p.Hkv, (unsigned)p.S);
#define QUOKA_ATTN(D)                                                                       \
  hipLaunchKernelGGL((attn_mfma_kernel<D>), grid, dim3(256), 0, st, (const bf16*)q,         \
                     (const bf16*)k_sel, (const bf16*)v_sel, (const bf16*)k_chunk,          \
                     (const bf16*)v_chunk, p.cu_chunk, p.cu_hist, p.Hq, p.Hkv, p.G,         \
                     p.kv_budget, sl2, (bf16*)out)
    if (p.D == 128) QUOKA_ATTN(128); else QUOKA_ATTN(64);
#undef QUOKA_ATTN
  } else {
    dim3 grid((unsigned)((p.maxC + 63) / 64), (unsigned)p.Hq, (unsigned)p.S);
#define QUOKA_ATTN(D)                                                                       \
  hipLaunchKernelGGL((attn_valu_kernel<float, D>), grid, dim3(64), 0, st, (const float*)q,  \
                     (const float*)k_sel, (const float*)v_sel, (const float*)k_chunk,       \
                     (const float*)v_chunk, p.cu_chunk, p.cu_hist, p.Hq, p.Hkv, p.G,        \
                     p.kv_budget, sl2, (float*)out)
    if (p.D == 128) QUOKA_ATTN(128); else QUOKA_ATTN(64);
#undef QUOKA_ATTN
  }
  return hipGetLastError();
}

}  // namespace quoka
