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

#include <type_traits>

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
    const int32_t* __restrict__ sel, const T* __restrict__ k_chunk, const T* __restrict__ v_chunk,
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
  const int L_off = cu_hist[s];
  const int L = cu_hist[s + 1] - L_off;
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
    // history rows: kept rows of k_sel / v_sel, or (sel given) rows sel[b] of
    // this sequence's k_hist / v_hist passed in their place
    const bool indexed = phase == 0 && sel != nullptr;
    const T* kb = phase == 1 ? k_chunk + ((int64_t)c_off * Hkv + h) * D
                  : indexed ? k_sel + ((int64_t)L_off * Hkv + h) * D : k_sel + prob * kv_budget * D;
    const T* vb = phase == 1 ? v_chunk + ((int64_t)c_off * Hkv + h) * D
                  : indexed ? v_sel + ((int64_t)L_off * Hkv + h) * D : v_sel + prob * kv_budget * D;
    const int64_t stride = (phase == 0 && !indexed) ? D : (int64_t)Hkv * D;
    for (int k0 = 0; k0 < nkeys; k0 += KT) {
      __syncthreads();
      for (int idx = lane; idx < KT * D; idx += 64) {
        const int r = idx / D, c = idx % D;
        int row = k0 + r;
        bool ok = row < nkeys;
        if (indexed && ok) {
          row = sel[prob * kv_budget + row];
          ok = (unsigned)row < (unsigned)L;
        }
        Ks[r][c] = ok ? to_f32(kb[(int64_t)row * stride + c]) : 0.f;
        Vs[r][c] = ok ? to_f32(vb[(int64_t)row * stride + c]) : 0.f;
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
// A workgroup of NW waves (4 or 8) owns NW*32 packed query rows of one
// (sequence, KV head); row r is token r / G, query head h*G + r % G, so the G
// heads that share the KV head share every K/V tile. Each wave owns 32 rows.
//   S^T = K Q^T  : A = K tile rows from LDS, B = the wave's Q held in VGPRs,
//                  C lane l = query column l%32, 16 key rows.
//   O^T += V^T P^T: A = V^T via LDS transpose reads of row-major V, B = P taken straight
//                  from the S^T accumulators; the 16 keys of a k-step are the
//                  ones the lane already holds, so P never leaves registers.
//                  Row sums are dot products of the bf16 P pairs.
// K/V tiles of 64 keys: first the kept history (masked past B_eff), then the
// chunk's keys up to the workgroup's last token (causal mask per row, only
// on tiles that reach past a wave's first token). LDS is double buffered:
// while a tile is consumed, the next one is in flight from HBM/L2 straight
// into the other buffer (buffer loads that write LDS, no register staging;
// an out-of-range load writes zeros); one barrier per tile.
// Blocks are renumbered so that all tiles of one KV head run on one XCD
// (blocks are dealt round-robin to the 8 XCDs) and share its L2.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

constexpr int kAttnKeys = 64;  // keys per K/V tile
constexpr int64_t kAttnMaxSplit = 8;  // key ranges per row tile, at most

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 4-element reads of group lanes i/4, i/4+4, i/4+8, i/4+12. With group
// lane j pointing at V[k0 + j/4][d0 + 4 (j%4)], lane i gets V[k0 .. k0+3][d0 + i]:
// four consecutive keys of one d, the A-operand slice of V^T.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  return __builtin_bit_cast(bf16x4, v);
}

// Logical id of this block: linear block L runs on XCD L % 8, and XCD x is
// given a contiguous range of logical ids (so a KV head's tiles share an L2).
__device__ __forceinline__ int xcd_logical_block(int nblk) {
  const int L = blockIdx.x;
  const int qx = nblk / kXcds, rx = nblk % kXcds, x = L % kXcds, slot = L / kXcds;
  return x < rx ? x * (qx + 1) + slot : rx * (qx + 1) + (x - rx) * qx + slot;
}

// LDS slot of the 16-byte chunk c of K/V tile row r: c ^ k(r) for K, c ^ v(r)
// for V. LDS serves 64 4-byte banks; a 16-byte read takes 16 lanes at a time
// and an 8-byte transposing read 32, and a group whose lanes share a bank
// pays an extra cycle (both measured on the chip: with c ^ (r & 7) every K
// read of 16 rows paid 4 extra cycles, with c ^ 2(r & 3) every V read of
// 4 rows x 4 chunks 2). K: a read of 16 rows (one chunk each) covers all 64
// banks. V, kR16 = false: a 32-lane transposing read of 4 rows x 4 chunks
// (32 rows per wave); kR16 = true: of 8 rows x 2 chunks (16 rows per wave).
template <int D, bool kR16>
struct KVSwizzle {
  __device__ static int k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int v(int r) {
    if constexpr (kR16) return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
    else return D == 128 ? 4 * (r & 3) : 2 * (r & 3);
  }
};

// The K/V tiles of one (sequence, KV head) for a workgroup of NW waves, 64
// keys per tile: first the kept history (k_sel / v_sel rows, or with kIdx the
// rows of k_hist / v_hist that the kept indices name: the gather fused in),
// then the chunk's own keys up to the workgroup's last token t_last. Tiles
// arrive by buffer loads that write LDS directly (a wave instruction fills
// 1 KB, lane l at +16 l, i.e. RPP rows of CPR 16-byte chunks; lane l of piece
// P takes row P*RPP + l/CPR and fetches the chunk that belongs in slot l%CPR),
// so no registers stage them; reads past the valid rows (the tail past B_eff,
// index -1) fall outside the buffer resource and write zeros. With kIdx the
// history row indices are fetched one tile ahead, so that a row load never
// waits for its own index load.
template <int D, int NW, bool kIdx, bool kR16>
struct KVTiles {
  static constexpr int KT = kAttnKeys, CPR = D / 8, RPP = 64 / CPR, NP = KT / RPP / NW;
  static_assert(NP >= 1 && KT % (RPP * NW) == 0, "tile must split into whole pieces per wave");
  using Swz = KVSwizzle<D, kR16>;
  using lds_ptr = __attribute__((address_space(3))) void*;
  const bf16 *k1, *v1, *k2, *v2;
  const int32_t* sidx;
  uint32_t rb1, rb2, end1, end2;
  int n1, B_eff, Lh, wave;
  int prow[NP], nidx[NP];
  uint32_t kcol[NP], vcol[NP];

  __device__ __forceinline__ KVTiles(const bf16* k_sel, const bf16* v_sel, const int32_t* sel,
                                     const bf16* k_chunk, const bf16* v_chunk, int s, int h,
                                     int Hkv, int c_off, int h_off, int Lh_, int kv_budget,
                                     int t_last, int wave_) {
    const int64_t prob = (int64_t)s * Hkv + h;
    Lh = Lh_;
    B_eff = min(kv_budget, Lh);
    wave = wave_;
    k1 = kIdx ? k_sel + ((int64_t)h_off * Hkv + h) * D : k_sel + prob * kv_budget * D;
    v1 = kIdx ? v_sel + ((int64_t)h_off * Hkv + h) * D : v_sel + prob * kv_budget * D;
    k2 = k_chunk + ((int64_t)c_off * Hkv + h) * D;
    v2 = v_chunk + ((int64_t)c_off * Hkv + h) * D;
    n1 = (B_eff + KT - 1) / KT;
    rb1 = kIdx ? (uint32_t)Hkv * D * 2u : D * 2u;  // row bytes
    rb2 = (uint32_t)Hkv * D * 2u;
    end1 = kIdx ? (Lh > 0 ? (uint32_t)(Lh - 1) * rb1 + D * 2u : 0u)  // valid bytes
                : (uint32_t)B_eff * rb1;
    end2 = (uint32_t)t_last * rb2 + D * 2u;
    sidx = sel + prob * kv_budget;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int r = (wave * NP + u) * RPP + lane / CPR, sl = lane % CPR;
      prow[u] = r;
      kcol[u] = (uint32_t)(sl ^ Swz::k(r)) * 16u;
      vcol[u] = (uint32_t)(sl ^ Swz::v(r)) * 16u;
    }
  }
  // history row indices of tile it
  __device__ __forceinline__ void fetch_idx(int it) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int key = it * KT + prow[u];
      nidx[u] = key < B_eff ? sidx[key] : -1;
    }
  }
  // tile it into kd / vd (with kIdx, tile it's indices fetched beforehand)
  __device__ __forceinline__ void load(int it, bf16* kd, bf16* vd) {
    const bool ph1 = it < n1;
    const int kbase = (ph1 ? it : it - n1) * KT;
    if (kIdx && ph1) {
      // row of key kbase + r is history row sel[kbase + r]; padding (-1) and
      // out-of-range indices read at the end of the buffer, i.e. as zeros
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(k1, end1), rv = make_rsrc(v1, end1);
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int row = nidx[u];
        const bool ok = (unsigned)row < (unsigned)Lh;
        const uint32_t base = (uint32_t)row * rb1;
        bf16* kp = kd + (wave * NP + u) * 512;
        bf16* vp = vd + (wave * NP + u) * 512;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)kp, 16, (int)(ok ? base + kcol[u] : end1), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)vp, 16, (int)(ok ? base + vcol[u] : end1), 0, 0, 0);
      }
      if (it + 1 < n1) fetch_idx(it + 1);
      return;
    }
    const uint32_t rb = ph1 ? rb1 : rb2;
    const uint32_t skip = (uint32_t)kbase * rb;
    const uint32_t left = (ph1 ? end1 : end2) - skip;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((ph1 ? k1 : k2) + (int64_t)kbase * (rb / 2), left);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((ph1 ? v1 : v2) + (int64_t)kbase * (rb / 2), left);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const uint32_t base = (uint32_t)prow[u] * rb;
      bf16* kp = kd + (wave * NP + u) * 512;
      bf16* vp = vd + (wave * NP + u) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr)kp, 16, (int)(base + kcol[u]), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr)vp, 16, (int)(base + vcol[u]), 0, 0, 0);
    }
  }
};

template <int D, int NW, bool kIdx>
__global__ __launch_bounds__(NW * 64, (NW == 4 ? 2 : 1)) void attn_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_sel, const bf16* __restrict__ v_sel,
    const int32_t* __restrict__ sel, const bf16* __restrict__ k_chunk, const bf16* __restrict__ v_chunk,
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist, int S, int Hq,
    int Hkv, int G, int kv_budget, int ntile_max, int pair_order, float scale_log2,
    int nsplit, float* __restrict__ part_o, float2* __restrict__ part_ml, bf16* __restrict__ out) {
  constexpr int KT = kAttnKeys, NDS = D / 16, NDB = D / 32;
  // K and V tiles land straight from global memory (buffer loads into LDS),
  // two buffers each, unpadded 2D-byte rows with XOR-swizzled 16-byte chunks
  __shared__ __attribute__((aligned(1024))) bf16 Ks0[KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Ks1[KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs0[KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs1[KT * D];

  // logical ids: key range fastest, then tile, then head, then sequence;
  // ntile_max counts (tile, key range) units
  const int logical = xcd_logical_block(ntile_max * Hkv * S);
  const int bxs = logical % ntile_max;
  const int bx = bxs / nsplit, sigma = bxs % nsplit;
  const int h = (logical / ntile_max) % Hkv;
  const int s = logical / (ntile_max * Hkv);

  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int rows = C * G;
  // Rows come in 128-row tiles of four waves; an eight-wave workgroup takes
  // two of them. Longest rows (most keys) first, except that with pair_order
  // an eight-wave workgroup takes the u-th tile from the end and the u-th
  // from the start: the K/V tiles they share are loaded once, the light half
  // stops computing when its rows run out of keys, and every workgroup gets
  // the same amount of work.
  constexpr int NH = NW / 4;  // 128-row tiles per workgroup
  const int n128 = (rows + 127) / 128;
  const int nunit = (n128 + NH - 1) / NH;
  if (bx >= nunit) return;
  int th[NH];  // each half's 128-row tile, -1 = none
  if constexpr (NH == 1) {
    th[0] = nunit - 1 - bx;
  } else if (pair_order) {
    th[0] = n128 - 1 - bx;
    th[1] = bx < n128 - 1 - bx ? bx : -1;
  } else {
    const int u = nunit - 1 - bx;
    th[0] = 2 * u;
    th[1] = 2 * u + 1 < n128 ? 2 * u + 1 : -1;
  }
  const int h_off = cu_hist[s];
  const int Lh = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, Lh);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int col = lane & 31, hi = lane >> 5;
  const int my_tile = th[wave / 4];
  const int row0 = max(my_tile, 0) * 128 + (wave % 4) * 32;  // the wave's first row
  const bool wave_live = my_tile >= 0 && row0 < rows;
  const int r = row0 + col;
  const bool rvalid = wave_live && r < rows;
  const int t = rvalid ? r / G : 0;
  const int jh = h * G + (rvalid ? r % G : 0);
  const int t_wave_first = min(C - 1, row0 / G);
  const int t_wave_last = min(C - 1, (row0 + 31) / G);

  bf16x8 qreg[NDS];
  {
    const bf16* qrow = q + ((int64_t)(c_off + t) * Hq + jh) * D + hi * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 v = *(const bf16x8*)(qrow + ds * 16);
      qreg[ds] = rvalid ? v : (bf16x8){};
    }
  }
  int top = th[0];
#pragma unroll
  for (int i = 1; i < NH; ++i) top = max(top, th[i]);
  const int t_last = min(C - 1, (top * 128 + 127) / G);  // the workgroup's last token
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY, l_part = 0.f;

  KVTiles<D, NW, kIdx, false> kv(k_sel, v_sel, sel, k_chunk, v_chunk, s, h, Hkv, c_off, h_off,
                                  Lh, kv_budget, t_last, wave);
  const int n1 = kv.n1;
  const int n_all = n1 + (t_last + KT) / KT;
  // with nsplit > 1 this workgroup takes the sigma-th of nsplit near-equal
  // ranges of the n_all key tiles
  const int it0 = (int)((int64_t)sigma * n_all / nsplit);
  const int it1 = (int)((int64_t)(sigma + 1) * n_all / nsplit);
  using Swz = KVSwizzle<D, false>;
  if (kIdx && it0 < n1) kv.fetch_idx(it0);
  if (it0 < it1) kv.load(it0, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // lane-constant parts of the LDS read addresses
  const int g16 = lane >> 4, j16 = lane & 15;
  // K operand of d-step ds: row sb*32 + col, chunk 2 ds + hi stored at
  // slot (2 ds + hi) ^ k(col) (sb*32 leaves the swizzle unchanged)
  int koff[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) koff[ds] = col * D + (((2 * ds + hi) ^ Swz::k(col)) << 3);
  // V transpose reads: row hi*4 + j16/4 (+ tile offsets, all multiples of 8,
  // which leave the swizzle unchanged), columns db*32 + (g16&1)*16 + 4(j16&3);
  // chunk c sits at c ^ v(row)
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int c = db * 4 + (g16 & 1) * 2 + ((j16 & 3) >> 1);
    const int row = hi * 4 + (j16 >> 2);
    voff[db] = row * D + ((c ^ Swz::v(row)) << 3) + 4 * (j16 & 1);
  }
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};

  auto step = [&, B_eff, t_wave_first, t_wave_last, n1, it1, t](int it, auto Bc)
                  __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    bf16* kcur = B ? Ks1 : Ks0;
    bf16* vcur = B ? Vs1 : Vs0;
    if (it + 1 < it1) kv.load(it + 1, B ? Ks0 : Ks1, B ? Vs0 : Vs1);
    const bool ph1 = it < n1;
    const int kbase = (ph1 ? it : it - n1) * KT;
    const bf16* ks = kcur;
    const bf16* vs = vcur;
    // a wave without rows, or whose rows' tokens all precede this chunk
    // tile, only helps with the loads
    if (wave_live && (ph1 || kbase <= t_wave_last)) {
    // S^T = K Q^T for the 64 keys of the tile (two 32-key blocks, interleaved)
    f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
    // all 16 K operands are read before the MFMAs so LDS latency overlaps
    bf16x8 ka[2][NDS];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        ka[sb][ds] = *(const bf16x8*)(ks + sb * 32 * D + koff[ds]);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[sb][ds], qreg[ds], sacc[sb], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
    // masks: history tail past B_eff; causal on tiles reaching past the
    // wave's first token
    const bool need_mask = ph1 ? (kbase + KT > B_eff) : (kbase + KT - 1 > t_wave_first);
    if (need_mask) {
      const int lim = (ph1 ? B_eff - 1 : t) - kbase - hi * 4;  // visible: key offset <= lim
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            if (sb * 32 + jj + 8 * i > lim) sacc[sb][i * 4 + jj] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[sb][e]);
    // max across the two lane halves that hold the same query column
    { const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
      mx = fmaxf(mx, fmaxf(__int_as_float(pr[0]), __int_as_float(pr[1]))); }
    // lazy rescaling: the reference max moves only when the tile's max
    // exceeds it by more than 32 in log2 units, so p <= 2^32 (fp32 and bf16
    // hold that with their usual relative precision; row sums stay far below
    // the fp32 range) and the output is rescaled on few tiles (exact either
    // way). On the channel-scaled layer data a bound of 8 rescaled often
    // enough to cost 2-5 % of the kernel.
    const float m_cand = fmaxf(m_run, mx);
    const bool upd = (m_cand - m_run) * scale_log2 > 32.0f;
    if (__ballot(upd)) {
      const float m_new = upd ? m_cand : m_run;
      const float alpha = upd ? __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2) : 1.f;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    // a row with no visible key yet (its key range starts past its token)
    // keeps p = 0 instead of exp2(-inf + inf)
    const float base = m_run == -INFINITY ? 0.f : m_run * scale_log2;
    bf16x8 pb[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[sb][i * 4 + jj], scale_log2, -base));
          pb[sb][i >> 1][(i & 1) * 4 + jj] = (bf16)p;
        }
    // row sums of the bf16 P actually multiplied, two keys per instruction
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 v = pb[sb][kk];
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, l_part, false);
      }
    // O^T += V^T P^T; the A operand is read transposed from row-major V: lane
    // group g = lane/16 covers d0 = db*32 + (g&1)*16, keys kb0 = ... + hi*4
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 a[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* p0 = vs + (sb * 32 + kk * 16) * D + voff[db];
          const bf16x4 lo4 = lds_read_tr16(p0);
          const bf16x4 hi4 = lds_read_tr16(p0 + 8 * D);
          a[db] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[db], pb[sb][kk], oacc[db], 0, 0, 0);
      }
    }
    // this wave's loads of the next tile have landed; after the barrier
    // every wave's have
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int it = it0; it < it1; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < it1) step(it + 1, std::integral_constant<int, 1>{});
  }

  uint32_t la, lb;
  swap32(__float_as_uint(l_part), la, lb);  // the two lane halves of each query column
  const float l_run = __uint_as_float(la) + __uint_as_float(lb);
  if (nsplit > 1) {
    // this key range's unnormalised state: O, and (reference max in log2
    // units, row sum), combined with the other ranges' by attn_merge_kernel
    if (rvalid) {
      const int64_t nrow = (int64_t)cu_chunk[S] * Hq;
      const int64_t grow = (int64_t)(c_off + t) * Hq + jh;
      float* po = part_o + ((int64_t)sigma * nrow + grow) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *(f32x4*)(po + db * 32 + hi * 4 + 8 * i) =
              (f32x4){oacc[db][i * 4], oacc[db][i * 4 + 1], oacc[db][i * 4 + 2], oacc[db][i * 4 + 3]};
      if (hi == 0)
        part_ml[sigma * nrow + grow] =
            make_float2(m_run == -INFINITY ? -INFINITY : m_run * scale_log2, l_run);
    }
    return;
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

// ---------------------------------------------------------------------------
// MFMA path with 16 rows per wave (v_mfma_f32_16x16x32_bf16), eight waves per
// 128-row tile: for shapes with at most one four-wave tile per CU, where the
// 32-row kernel leaves a single wave per SIMD to run its chain of dependent
// 64-key steps alone; here every SIMD holds two waves of half the work.
//   S^T = K Q^T : A = 16 keys x 32 d of the K tile (LDS), B = the wave's Q
//                 (registers); C lane l = query row l%16, keys (l/16)*4..+3
//                 of each 16-key block.
//   O^T += V^T P^T per 32-key step: B = P straight from the S^T accumulators
//                 of its two 16-key blocks (lane l holds keys (l/16)*4..+3 of
//                 each, which is the MFMA's k-slice (l/16)*8..+7 under a
//                 fixed permutation of the step's keys); A = V^T read
//                 transposed for the same permutation (two 4-key reads).
// Tile order, masks, lazy rescaling, loads and the fused gather are as in
// attn_mfma_kernel; V rows are swizzled so that each 32-lane group of a
// transposing read (8 keys x 2 chunks) covers all 64 banks once. Every wave
// reads the whole K and V tile for half the rows of the 32-row kernel, so the
// LDS carries twice the bytes per product: worth it only where the 32-row
// kernel has a single wave per SIMD (narrow layer: 53.6 -> 49.2 us; four-wave
// 64-row tiles, two per CU, measured the same 49.4 us).
// ---------------------------------------------------------------------------
template <int D, int NW, bool kIdx>
__global__ __launch_bounds__(NW * 64, (NW == 4 ? 2 : 1)) void attn_r16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_sel, const bf16* __restrict__ v_sel,
    const int32_t* __restrict__ sel, const bf16* __restrict__ k_chunk, const bf16* __restrict__ v_chunk,
    const int32_t* __restrict__ cu_chunk, const int32_t* __restrict__ cu_hist, int S, int Hq,
    int Hkv, int G, int kv_budget, int ntile_max, float scale_log2, bf16* __restrict__ out) {
  constexpr int KT = kAttnKeys, NDS = D / 32, NDB = D / 16, TR = NW * 16;  // TR rows per tile
  __shared__ __attribute__((aligned(1024))) bf16 Ks0[KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Ks1[KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs0[KT * D];
  __shared__ __attribute__((aligned(1024))) bf16 Vs1[KT * D];

  const int logical = xcd_logical_block(ntile_max * Hkv * S);
  const int bx = logical % ntile_max;
  const int h = (logical / ntile_max) % Hkv;
  const int s = logical / (ntile_max * Hkv);

  const int c_off = cu_chunk[s];
  const int C = cu_chunk[s + 1] - c_off;
  const int rows = C * G;
  const int ntr = (rows + TR - 1) / TR;
  if (bx >= ntr) return;
  const int tile = ntr - 1 - bx;  // longest rows (most keys) first
  const int h_off = cu_hist[s];
  const int Lh = cu_hist[s + 1] - h_off;
  const int B_eff = min(kv_budget, Lh);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15, g4 = lane >> 4;
  const int row0 = tile * TR + wave * 16;  // the wave's first row
  const bool wave_live = row0 < rows;
  const int r = row0 + rl;
  const bool rvalid = r < rows;
  const int t = rvalid ? r / G : 0;
  const int jh = h * G + (rvalid ? r % G : 0);
  const int t_wave_first = min(C - 1, row0 / G);
  const int t_wave_last = min(C - 1, (row0 + 15) / G);

  // B operand of S^T: lane l holds Q[row l%16][ds*32 + (l/16)*8 ..+7]
  bf16x8 qreg[NDS];
  {
    const bf16* qrow = q + ((int64_t)(c_off + t) * Hq + jh) * D + g4 * 8;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 v = *(const bf16x8*)(qrow + ds * 32);
      qreg[ds] = rvalid ? v : (bf16x8){};
    }
  }
  const int t_last = min(C - 1, (tile * TR + TR - 1) / G);  // the workgroup's last token
  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  KVTiles<D, NW, kIdx, true> kv(k_sel, v_sel, sel, k_chunk, v_chunk, s, h, Hkv, c_off, h_off,
                                 Lh, kv_budget, t_last, wave);
  const int n1 = kv.n1;
  const int n_all = n1 + (t_last + KT) / KT;
  using Swz = KVSwizzle<D, true>;
  if (kIdx && 0 < n1) kv.fetch_idx(0);
  if (0 < n_all) kv.load(0, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // K operand of (key block kb, d-step ds): row kb*16 + l%16, chunk
  // ds*4 + l/16 (kb*16 leaves the swizzle unchanged)
  int koff[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) koff[ds] = rl * D + (((ds * 4 + g4) ^ Swz::k(rl)) << 3);
  // V^T operand of d-block db: 16-lane group g reads keys g*4 + j/4 (+16 for
  // the second half of the step), columns db*16 + 4 (j%4), j = l%16
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int row = g4 * 4 + (rl >> 2);
    const int c = db * 2 + ((rl & 3) >> 1);
    voff[db] = row * D + ((c ^ Swz::v(row)) << 3) + 4 * (rl & 1);
  }
  const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};

  auto step = [&](int it, auto Bc) __attribute__((always_inline)) {
    constexpr int B = decltype(Bc)::value;
    const bf16* ks = B ? Ks1 : Ks0;
    const bf16* vs = B ? Vs1 : Vs0;
    if (it + 1 < n_all) kv.load(it + 1, B ? Ks0 : Ks1, B ? Vs0 : Vs1);
    const bool ph1 = it < n1;
    const int kbase = (ph1 ? it : it - n1) * KT;
    if (wave_live && (ph1 || kbase <= t_wave_last)) {
      f32x4 sacc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[kb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        bf16x8 ka[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) ka[kb] = *(const bf16x8*)(ks + kb * 16 * D + koff[ds]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kb], qreg[ds], sacc[kb], 0, 0, 0);
      }
      const bool need_mask = ph1 ? (kbase + KT > B_eff) : (kbase + KT - 1 > t_wave_first);
      if (need_mask) {
        const int lim = (ph1 ? B_eff - 1 : t) - kbase - g4 * 4;  // visible: offset <= lim
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb * 16 + e > lim) sacc[kb][e] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        mx = fmaxf(mx, fmaxf(fmaxf(sacc[kb][0], sacc[kb][1]), fmaxf(sacc[kb][2], sacc[kb][3])));
      mx = rows_max(mx);  // the four lanes of the row
      const float m_cand = fmaxf(m_run, mx);
      const bool upd = (m_cand - m_run) * scale_log2 > 32.0f;
      if (__ballot(upd)) {
        const float m_new = upd ? m_cand : m_run;
        const float alpha = upd ? __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      const float base = m_run == -INFINITY ? 0.f : m_run * scale_log2;
      // P of the 32-key step ks: keys g*4..+3 of block 2ks, then of block 2ks + 1
      bf16x8 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pb[ks][e] = (bf16)__builtin_amdgcn_exp2f(
              fmaf(sacc[2 * ks + (e >> 2)][e & 3], scale_log2, -base));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 v = pb[ks];
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one2, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one2, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one2, l_part, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one2, l_part, false);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 a[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16* p0 = vs + ks * 32 * D + voff[db];
          const bf16x4 lo4 = lds_read_tr16(p0);
          const bf16x4 hi4 = lds_read_tr16(p0 + 16 * D);
          a[db] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[db], pb[ks], oacc[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int it = 0; it < n_all; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < n_all) step(it + 1, std::integral_constant<int, 1>{});
  }

  const float l_run = rows_sum(l_part);
  if (rvalid) {
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    bf16* orow = out + ((int64_t)(c_off + t) * Hq + jh) * D + g4 * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (bf16)(oacc[db][e] * inv);
      *(bf16x4*)(orow + db * 16) = v;
    }
  }
}

// Combination of the key ranges' states of a row (the online softmax's merge
// step): with b = the largest reference max (log2 units),
// O = sum_r 2^(b_r - b) O_r / sum_r 2^(b_r - b) l_r. A range that saw no key
// of the row (b_r = -inf) adds nothing. One thread per 8 outputs of a row.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         int nsplit, int64_t nrow,
                                                         bf16* __restrict__ out) {
  constexpr int CPR = D / 8;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = i / CPR;
  const int c = (int)(i % CPR);
  if (row >= nrow) return;
  float b = -INFINITY;
  for (int r = 0; r < nsplit; ++r) b = fmaxf(b, part_ml[r * nrow + row].x);
  float l = 0.f;
  f32x4 a0 = {}, a1 = {};
  for (int r = 0; r < nsplit; ++r) {
    const float2 ml = part_ml[r * nrow + row];
    if (ml.x == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(ml.x - b);
    l = fmaf(w, ml.y, l);
    const f32x4* po = (const f32x4*)(part_o + (r * nrow + row) * D + c * 8);
    a0 += w * po[0];
    a1 += w * po[1];
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (bf16)(a0[e] * inv);
    v[4 + e] = (bf16)(a1[e] * inv);
  }
  *(bf16x8*)(out + row * D + c * 8) = v;
}

// Eight-wave workgroups share each K/V tile between twice the rows (half the
// LDS writes and L2 reads per row) but hold twice the rows, so a shape has
// half as many of them; they are used when that still leaves two per CU
// (with one per CU, the causal spread of work between tiles is exposed).
constexpr int kAttnWideMinBlocks = 512;
// Four-wave workgroups resident at once on the chip: two per CU (LDS and
// registers), 256 CUs.
constexpr int kAttnResident4 = 2 * 256;

namespace {

struct AttnPlan {
  int nw, pair, ntile, nsplit;
  bool r16;  // 16 rows per wave (attn_r16_kernel)
};

AttnPlan attn_plan(const Problem& p) {
  const int64_t rows = (int64_t)p.maxC * p.G;
  const int64_t n128 = (rows + 127) / 128;
  const int64_t grid4 = n128 * p.Hkv * p.S;  // four-wave workgroups the shape needs
  // Eight waves on a heavy and a light 128-row tile (the paired order: every
  // workgroup gets the same work and its halves share the K/V loads) when
  // four-wave workgroups would fill the chip exactly once, or when there are
  // enough for eight-wave workgroups and the chunk spans at most half as many
  // key tiles as the kept history (the light half then idles only briefly:
  // ragged layer 112 -> 107 us); eight waves on 256 contiguous rows when
  // there are enough for them and the chunk is longer (long layer: the
  // paired order's light halves idled, 406 -> 415 us); else four waves.
  const bool many = (rows + 255) / 256 * p.Hkv * p.S >= kAttnWideMinBlocks;
  const int64_t hist_tiles = (p.kv_budget + 63) / 64, chunk_tiles = (p.maxC + 63) / 64;
  const bool short_chunk = chunk_tiles * 2 <= hist_tiles;
  const bool wide = many && !short_chunk;
  const int pair =
      ((!many && grid4 > 256 && grid4 <= kAttnResident4) || (many && short_chunk)) ? 1 : 0;
  const int nw = (wide || pair) ? 8 : 4;
  const int ntile = (int)(nw == 8 ? (n128 + 1) / 2 : n128);
  // at most half the CUs busy (few rows: short chunks, decode): split each
  // tile's key tiles into ranges, about one workgroup per CU, and merge the
  // ranges' states afterwards. Measured on the narrow layer (224 workgroups)
  // a split gained nothing: the partial states' HBM round trip cost what the
  // balance won, so the rule stops at half the chip.
  int nsplit = 1;
  if (nw == 4 && grid4 <= 128) {
    const int64_t steps = (p.kv_budget + 63) / 64 + (p.maxC + 63) / 64;
    nsplit = (int)std::max<int64_t>(1, std::min<int64_t>({256 / grid4, steps, kAttnMaxSplit}));
  }
  // at most one four-wave tile per CU and no key split: sixteen rows per wave,
  // eight waves per tile, so that every SIMD runs two waves
  const bool r16 = nw == 4 && nsplit == 1 && grid4 <= 256;
  return {nw, pair, ntile, nsplit, r16};
}

}  // namespace

void attn_describe(const Problem& p, int* kernel, int* key_ranges) {
  if (p.dtype != QUOKA_BF16) {
    *kernel = QUOKA_ATTN_VALU;
    *key_ranges = 1;
    return;
  }
  const AttnPlan a = attn_plan(p);
  *kernel = a.r16 ? QUOKA_ATTN_ROWS16
          : a.nw == 4 ? QUOKA_ATTN_ROWS32_4W
          : a.pair ? QUOKA_ATTN_ROWS32_8W_PAIRED : QUOKA_ATTN_ROWS32_8W;
  *key_ranges = a.nsplit;
}

size_t attn_workspace_bytes(const Problem& p) {
  if (p.dtype != QUOKA_BF16 || p.maxC == 0) return 0;
  const AttnPlan a = attn_plan(p);
  if (a.nsplit == 1) return 0;
  const size_t nrow = (size_t)p.TC * p.Hq;
  return (size_t)a.nsplit * nrow * ((size_t)p.D * 4 + 8);
}

hipError_t launch_attention(const Problem& p, const void* q, const void* k_sel,
                            const void* v_sel, const int32_t* sel, const void* k_chunk,
                            const void* v_chunk, float scale, void* out, void* attn_ws,
                            hipStream_t st) {
  if (p.maxC == 0) return hipSuccess;
  const float sl2 = scale * kLog2e;
  if (p.dtype == QUOKA_BF16) {
    const AttnPlan a = attn_plan(p);
    const int nw = a.nw, pair = a.pair, ntile = a.ntile, nsplit = a.nsplit;
    const int64_t nrow = (int64_t)p.TC * p.Hq;
    float* part_o = nullptr;
    float2* part_ml = nullptr;
    if (nsplit > 1) {
      if (!attn_ws) return hipErrorInvalidValue;
      part_o = (float*)attn_ws;
      part_ml = (float2*)(part_o + (size_t)nsplit * nrow * p.D);
    }
    dim3 grid((unsigned)(ntile * nsplit * p.Hkv * p.S));
#define QUOKA_ATTN(D, NW, IDX)                                                                 \
  hipLaunchKernelGGL((attn_mfma_kernel<D, NW, IDX>), grid, dim3(NW * 64), 0, st, (const bf16*)q, \
                     (const bf16*)k_sel, (const bf16*)v_sel, sel, (const bf16*)k_chunk,           \
                     (const bf16*)v_chunk, p.cu_chunk, p.cu_hist, p.S, p.Hq, p.Hkv, p.G,          \
                     p.kv_budget, ntile * nsplit, pair, sl2, nsplit, part_o, part_ml, (bf16*)out)
#define QUOKA_ATTN_R16(D, IDX)                                                                 \
  hipLaunchKernelGGL((attn_r16_kernel<D, 8, IDX>), grid, dim3(512), 0, st, (const bf16*)q,      \
                     (const bf16*)k_sel, (const bf16*)v_sel, sel, (const bf16*)k_chunk,           \
                     (const bf16*)v_chunk, p.cu_chunk, p.cu_hist, p.S, p.Hq, p.Hkv, p.G,          \
                     p.kv_budget, ntile, sl2, (bf16*)out)
#define QUOKA_ATTN_NW(D, IDX) { if (a.r16) QUOKA_ATTN_R16(D, IDX); else if (nw == 8) QUOKA_ATTN(D, 8, IDX); else QUOKA_ATTN(D, 4, IDX); }
    if (sel) { if (p.D == 128) QUOKA_ATTN_NW(128, true) else QUOKA_ATTN_NW(64, true) }
    else     { if (p.D == 128) QUOKA_ATTN_NW(128, false) else QUOKA_ATTN_NW(64, false) }
#undef QUOKA_ATTN_NW
#undef QUOKA_ATTN_R16
#undef QUOKA_ATTN
    if (nsplit > 1) {
      const int64_t nthr = nrow * (p.D / 8);
      dim3 mg((unsigned)((nthr + 255) / 256));
      if (p.D == 128)
        hipLaunchKernelGGL(attn_merge_kernel<128>, mg, dim3(256), 0, st, part_o, part_ml, nsplit,
                           nrow, (bf16*)out);
      else
        hipLaunchKernelGGL(attn_merge_kernel<64>, mg, dim3(256), 0, st, part_o, part_ml, nsplit,
                           nrow, (bf16*)out);
    }
  } else {
    dim3 grid((unsigned)((p.maxC + 63) / 64), (unsigned)p.Hq, (unsigned)p.S);
#define QUOKA_ATTN(D)                                                                       \
  hipLaunchKernelGGL((attn_valu_kernel<float, D>), grid, dim3(64), 0, st, (const float*)q,  \
                     (const float*)k_sel, (const float*)v_sel, sel, (const float*)k_chunk, \
                     (const float*)v_chunk, p.cu_chunk, p.cu_hist, p.Hq, p.Hkv, p.G,        \
                     p.kv_budget, sl2, (float*)out)
    if (p.D == 128) QUOKA_ATTN(128); else QUOKA_ATTN(64);
#undef QUOKA_ATTN
  }
  return hipGetLastError();
}

}  // namespace quoka
