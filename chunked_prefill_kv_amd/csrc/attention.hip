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
// K/V tiles of 64 keys: first the kept history (masked past B_eff), then the
// chunk's keys up to the workgroup's last token (causal mask per row, only
// on tiles that reach past a wave's first token). LDS is double buffered:
// while a tile is consumed, the next one is in flight from HBM/L2 into VGPRs
// and lands in the other buffer; one barrier per tile.
// Blocks are renumbered so that all tiles of one KV head run on one XCD
// (blocks are dealt round-robin to the 8 XCDs) and share its L2.
// ---------------------------------------------------------------------------
constexpr int kAttnRows = 128;
constexpr int kXcds = 8;

template <int D>
struct AttnTile {
  static constexpr int KT = 64;                  // keys per tile
  static constexpr int KSTR = D + 8;             // K row stride in LDS (elements)
  static constexpr int VSTR = KT + 8;            // V^T row stride in LDS (elements)
  static constexpr int KCH = KT * D / 8 / 256;   // 16-byte K chunks per thread
  static constexpr int KPT = D / 32;             // V keys per thread (x 8 d-values)
  static constexpr int K_ELEMS = KT * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
};

template <int D>
__device__ __forceinline__ void attn_load_tile(const bf16* __restrict__ kp,
                                               const bf16* __restrict__ vp, int64_t rstride,
                                               int kbase, int klim, bf16x8 (&kr)[AttnTile<D>::KCH],
                                               bf16x8 (&vr)[AttnTile<D>::KPT]) {
  using TT = AttnTile<D>;
#pragma unroll
  for (int i = 0; i < TT::KCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / (D / 8), part = c % (D / 8);
    const int key = kbase + row;
    const bf16x8 v = *(const bf16x8*)(kp + (int64_t)(key < klim ? key : 0) * rstride + part * 8);
    kr[i] = key < klim ? v : (bf16x8){};
  }
  const int dg = threadIdx.x % (D / 8), kq = threadIdx.x / (D / 8);
#pragma unroll
  for (int i = 0; i < TT::KPT; ++i) {
    const int key = kbase + kq * TT::KPT + i;
    const bf16x8 v = *(const bf16x8*)(vp + (int64_t)(key < klim ? key : 0) * rstride + dg * 8);
    vr[i] = key < klim ? v : (bf16x8){};
  }
}

template <int D>
__device__ __forceinline__ void attn_store_tile(bf16* __restrict__ Ks, bf16* __restrict__ Vt,
                                                const bf16x8 (&kr)[AttnTile<D>::KCH],
                                                const bf16x8 (&vr)[AttnTile<D>::KPT]) {
  using TT = AttnTile<D>;
#pragma unroll
  for (int i = 0; i < TT::KCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int row = c / (D / 8), part = c % (D / 8);
    *(bf16x8*)&Ks[row * TT::KSTR + part * 8] = kr[i];
  }
  // V^T: this thread holds KPT consecutive keys x 8 consecutive d-values;
  // each d-row gets its KPT keys in one store.
  const int dg = threadIdx.x % (D / 8), kq = threadIdx.x / (D / 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16* dst = &Vt[(dg * 8 + e) * TT::VSTR + kq * TT::KPT];
    if constexpr (TT::KPT == 4) {
      bf16x4 t = {vr[0][e], vr[1][e], vr[2][e], vr[3][e]};
      *(bf16x4*)dst = t;
    } else {
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      bf16x2 t = {vr[0][e], vr[1][e]};
      *(bf16x2*)dst = t;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_sel, const bf16* __restrict__ v_sel,
    const bf16* __restrict__ k_chunk, const bf16* __restrict__ v_chunk,
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist, int S, int Hq,
    int Hkv, int G, int kv_budget, int ntile_max, float scale_log2, bf16* __restrict__ out) {
  using TT = AttnTile<D>;
  constexpr int KT = TT::KT, NDS = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][TT::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][TT::V_ELEMS];

  // XCD-aware renumbering: linear block L runs on XCD L % 8; give XCD x a
  // contiguous range of logical ids (tile-fastest, then head, then sequence).
  const int nblk = ntile_max * Hkv * S;
  const int L = blockIdx.x;
  const int qx = nblk / kXcds, rx = nblk % kXcds, x = L % kXcds, slot = L / kXcds;
  const int logical = x < rx ? x * (qx + 1) + slot : rx * (qx + 1) + (x - rx) * qx + slot;
  const int bx = logical % ntile_max;
  const int h = (logical / ntile_max) % Hkv;
  const int s = logical / (ntile_max * Hkv);

  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int rows = C * G;
  const int ntile = (rows + kAttnRows - 1) / kAttnRows;
  if (bx >= ntile) return;
  const int tile = ntile - 1 - bx;  // longest rows first
  const int h_off = cu_hist[s];
  const int Lh = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, Lh);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hi = lane >> 5;
  const int r = tile * kAttnRows + wave * 32 + col;
  const bool rvalid = r < rows;
  const int t = rvalid ? r / G : 0;
  const int jh = h * G + (rvalid ? r % G : 0);
  const int t_wave_first = min(C - 1, (tile * kAttnRows + wave * 32) / G);

  bf16x8 qreg[NDS];
  {
    const bf16* qrow = q + ((int64_t)(c_off + t) * Hq + jh) * D + hi * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 v = *(const bf16x8*)(qrow + ds * 16);
      qreg[ds] = rvalid ? v : (bf16x8){};
    }
  }
  const int t_last = min(C - 1, (tile * kAttnRows + kAttnRows - 1) / G);
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, l_part = 0.f;

  const int64_t prob = (int64_t)s * Hkv + h;
  const bf16* k1 = k_sel + prob * kv_budget * D;
  const bf16* v1 = v_sel + prob * kv_budget * D;
  const bf16* k2 = k_chunk + ((int64_t)c_off * Hkv + h) * D;
  const bf16* v2 = v_chunk + ((int64_t)c_off * Hkv + h) * D;
  const int n1 = (B_eff + KT - 1) / KT;
  const int n_all = n1 + (t_last + KT) / KT;

  bf16x8 kr[TT::KCH], vr[TT::KPT];
  auto load = [&](int it) {
    const bool ph1 = it < n1;
    const int kbase = (ph1 ? it : it - n1) * KT;
    attn_load_tile<D>(ph1 ? k1 : k2, ph1 ? v1 : v2, ph1 ? (int64_t)D : (int64_t)Hkv * D, kbase,
                      ph1 ? B_eff : t_last + 1, kr, vr);
  };
  load(0);
  attn_store_tile<D>(Ks[0], Vt[0], kr, vr);
  __syncthreads();

  for (int it = 0; it < n_all; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_all) load(it + 1);
    const bool ph1 = it < n1;
    const int kbase = (ph1 ? it : it - n1) * KT;
    const bf16* ks = Ks[buf];
    const bf16* vt = Vt[buf];

    f32x16 sacc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sacc[sb] = (f32x16){};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 a = *(const bf16x8*)&ks[(sb * 32 + col) * TT::KSTR + ds * 16 + hi * 8];
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], sacc[sb], 0, 0, 0);
      }
    }
    // masks: history tail past B_eff; causal on tiles reaching past the
    // wave's first token
    const bool need_mask = ph1 ? (kbase + KT > B_eff) : (kbase + KT - 1 > t_wave_first);
    if (need_mask) {
      const int lim = ph1 ? B_eff - 1 : t;  // visible keys: key <= lim
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int key = kbase + sb * 32 + hi * 4 + jj + 8 * i;
            if (key > lim) sacc[sb][i * 4 + jj] = -INFINITY;
          }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[sb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new > m_run ? exp2f((m_run - m_new) * scale_log2) : 1.f;
    const float base = m_new == -INFINITY ? 0.f : m_new * scale_log2;
    bf16x8 pb[2][2];
    float ps = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p = exp2f(fmaf(sacc[sb][i * 4 + jj], scale_log2, -base));
          ps += p;
          pb[sb][i >> 1][(i & 1) * 4 + jj] = (bf16)p;
        }
    l_part = fmaf(l_part, alpha, ps);
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16* vrow = vt + (db * 32 + col) * TT::VSTR;
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
    if (it + 1 < n_all) attn_store_tile<D>(Ks[buf ^ 1], Vt[buf ^ 1], kr, vr);
    __syncthreads();
  }

  const float l_run = l_part + __shfl_xor(l_part, 32, 64);
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
    const int ntile = (int)(((int64_t)p.maxC * p.G + kAttnRows - 1) / kAttnRows);
    dim3 grid((unsigned)(ntile * p.Hkv * p.S));
#define QUOKA_ATTN(D)                                                                       \
  hipLaunchKernelGGL((attn_mfma_kernel<D>), grid, dim3(256), 0, st, (const bf16*)q,         \
                     (const bf16*)k_sel, (const bf16*)v_sel, (const bf16*)k_chunk,          \
                     (const bf16*)v_chunk, p.cu_chunk, p.cu_hist, p.S, p.Hq, p.Hkv, p.G,    \
                     p.kv_budget, ntile, sl2, (bf16*)out)
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
