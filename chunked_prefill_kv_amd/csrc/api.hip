// C ABI of the QUOKA per-chunk hot path: argument validation, workspace
// layout and the launch sequence on the caller's stream. Declared and
// documented in include/quoka.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "common.h"
#include "debug.h"
#include "internal.h"
#include "quoka.h"

namespace quoka {

thread_local char g_err[512] = "";

quoka_status fail(quoka_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

namespace {

bool sync_mode() {
  static const bool on = [] {
    const char* v = std::getenv("QUOKA_SYNC");
    return v && v[0] && std::strcmp(v, "0") != 0;
  }();
  return on || debug_mode();
}

// QUOKA_DEBUG: the arguments' checks, run before a call's first compute
// kernel (debug.hip); nothing when the mode is off.
quoka_status debug_inputs(const Problem& p, std::initializer_list<DebugItem> items,
                          hipStream_t st) {
  if (!debug_mode()) return QUOKA_OK;
  const quoka_status rc = debug_offsets(p);
  if (rc != QUOKA_OK) return rc;
  return debug_run(p, items.begin(), (int)items.size(), st);
}

// element counts of the arguments
int64_t n_q(const Problem& p) { return p.TC * p.Hq * p.D; }
int64_t n_hist(const Problem& p) { return p.TL * p.Hkv * p.D; }
int64_t n_chunk(const Problem& p) { return p.TC * p.Hkv * p.D; }
int64_t n_sel(const Problem& p) { return (int64_t)p.S * p.Hkv * p.kv_budget; }

quoka_status hip_check(hipError_t e, const char* what, hipStream_t st) {
  if (e == hipSuccess && sync_mode()) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(QUOKA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return QUOKA_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest dynamic LDS the scorer asks for; raised once per device (the
// per-head baseline's kernels to all the device offers).
quoka_status ensure_lds(const Problem& p) {
  static std::mutex mu;
  static int max_lds[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QUOKA_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(QUOKA_EUNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (max_lds[dev] == 0) {
    int lds = 0;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return fail(QUOKA_EHIP, "hipDeviceGetAttribute(MaxSharedMemoryPerBlock) failed");
    const int need = kScoreBins * 4 + QUOKA_MAX_Q_BUDGET * 128 * 4;
    if (lds < need)
      return fail(QUOKA_EUNSUPPORTED,
                  "device offers %d bytes of LDS per workgroup, scorer needs %d", lds, need);
    const hipError_t e = set_scorer_lds_limit(need, lds);
    if (e != hipSuccess)
      return fail(QUOKA_EHIP, "hipFuncSetAttribute(scorer LDS): %s", hipGetErrorString(e));
    max_lds[dev] = lds;
  }
  const size_t want = scorer_lds_bytes(p);
  if (want > (size_t)max_lds[dev])
    return fail(QUOKA_EUNSUPPORTED,
                "the per-head baseline needs %zu bytes of LDS per workgroup, the device offers %d",
                want, max_lds[dev]);
  return QUOKA_OK;
}

// Scorer workgroups over all sequences for tiles of `keys` history keys.
int64_t scorer_tiles(const quoka_shape& sh, int keys) {
  int64_t n = 0;
  for (int s = 0; s < sh.num_seqs; ++s)
    n += ((int64_t)sh.cu_hist_host[s + 1] - sh.cu_hist_host[s] + keys - 1) / keys;
  return n;
}

quoka_status make_problem(const quoka_shape* sh, int q_budget, int kv_budget, Problem* p) {
  if (!sh) return fail(QUOKA_EINVAL, "shape is null");
  if (sh->num_seqs < 1) return fail(QUOKA_EINVAL, "num_seqs=%d must be >= 1", sh->num_seqs);
  if (sh->num_q_heads < 1 || sh->num_kv_heads < 1)
    return fail(QUOKA_EINVAL, "head counts must be >= 1 (H_q=%d, H_kv=%d)", sh->num_q_heads,
                sh->num_kv_heads);
  if (sh->num_q_heads % sh->num_kv_heads)
    return fail(QUOKA_EINVAL, "num_q_heads=%d is not a multiple of num_kv_heads=%d",
                sh->num_q_heads, sh->num_kv_heads);
  if (sh->dtype != QUOKA_F32 && sh->dtype != QUOKA_BF16)
    return fail(QUOKA_EINVAL, "dtype=%d is not a quoka_dtype", (int)sh->dtype);
  if (sh->head_dim != 64 && sh->head_dim != 128)
    return fail(QUOKA_EUNSUPPORTED, "head_dim=%d (built: 64, 128)", sh->head_dim);
  if (!sh->cu_chunk || !sh->cu_hist || !sh->cu_chunk_host || !sh->cu_hist_host)
    return fail(QUOKA_EINVAL, "cu_chunk / cu_hist device and host arrays must all be given");
  if (q_budget < 1) return fail(QUOKA_EINVAL, "q_budget=%d must be >= 1", q_budget);
  if (q_budget > QUOKA_MAX_Q_BUDGET)
    return fail(QUOKA_EUNSUPPORTED, "q_budget=%d exceeds %d", q_budget, QUOKA_MAX_Q_BUDGET);
  if (kv_budget < 1) return fail(QUOKA_EINVAL, "kv_budget=%d must be >= 1", kv_budget);
  const int S = sh->num_seqs;
  if (sh->cu_chunk_host[0] != 0 || sh->cu_hist_host[0] != 0)
    return fail(QUOKA_EINVAL, "cu_chunk_host[0] and cu_hist_host[0] must be 0");
  p->S = S;
  p->Hq = sh->num_q_heads;
  p->Hkv = sh->num_kv_heads;
  p->G = p->Hq / p->Hkv;
  p->D = sh->head_dim;
  p->dtype = sh->dtype;
  p->cu_chunk = sh->cu_chunk;
  p->cu_hist = sh->cu_hist;
  p->cu_chunk_h = sh->cu_chunk_host;
  p->cu_hist_h = sh->cu_hist_host;
  p->NQT = p->NSB = p->NKT = 0;
  p->maxC = p->maxL = 0;
  for (int s = 0; s < S; ++s) {
    const int64_t C = (int64_t)sh->cu_chunk_host[s + 1] - sh->cu_chunk_host[s];
    const int64_t L = (int64_t)sh->cu_hist_host[s + 1] - sh->cu_hist_host[s];
    if (C < 0 || L < 0)
      return fail(QUOKA_EINVAL, "cu offsets decrease at sequence %d", s);
    p->NKT += (L + kTopbKeys - 1) / kTopbKeys;
    p->maxC = std::max<int>(p->maxC, (int)C);
    p->maxL = std::max<int>(p->maxL, (int)L);
  }
  // Query-prep tiles of 64 tokens (4 per wave), or of 32 or 16 when that
  // leaves fewer workgroups than CUs (short chunks, few KV heads): the
  // query side then spreads over the chip instead of a few long workgroups.
  p->qtok = kQprepTokens;
  for (;;) {
    p->NQT = 0;
    for (int s = 0; s < S; ++s) {
      const int64_t C = (int64_t)sh->cu_chunk_host[s + 1] - sh->cu_chunk_host[s];
      p->NQT += (C + p->qtok - 1) / p->qtok;
    }
    if (p->qtok == kQprepTokens / 4 || p->NQT * p->Hkv >= 256) break;
    p->qtok /= 2;
  }
  // Scorer tiles: one 64-key block per wave while that takes at most two
  // rounds of workgroups; past that each wave streams several blocks with
  // the next one in flight, in tiles just large enough for a single round
  // (up to 2048 keys: beyond it the last workgroups' compute is exposed),
  // and no larger than it takes to lower the workgroup count (short
  // sequences).
  p->score_keys = kScoreKeysMin;
  p->NSB = scorer_tiles(*sh, p->score_keys);
  // With at most 32 kept rows (two 16-row blocks) a key block costs few
  // products and the scorer streams: tiles of 512 keys or more, the smallest
  // that gives at most two rounds (narrow layer 22.0 -> 20.3 us at 512 keys;
  // decode 59.3 -> 56.8 us at 1024 instead of 2048).
  if (std::min<int64_t>(q_budget, p->maxC) <= 32) {
    for (int k = 2 * kScoreKeysMin; k <= kScoreKeysMax; k *= 2) {
      const int64_t n = scorer_tiles(*sh, k);
      if (n * p->Hkv <= 2 * kScoreMaxBlocks) {
        p->score_keys = k;
        p->NSB = n;
        break;
      }
    }
  }
  if (p->NSB * p->Hkv > 2 * kScoreMaxBlocks) {
    while (p->score_keys < kScoreKeysMax && p->NSB * p->Hkv > kScoreMaxBlocks) {
      const int64_t n = scorer_tiles(*sh, p->score_keys * 2);
      if (n == p->NSB && p->score_keys > kScoreKeysMin) break;
      p->score_keys *= 2;
      p->NSB = n;
    }
  }
  p->TC = sh->cu_chunk_host[S];
  p->TL = sh->cu_hist_host[S];
  // element offsets are int64 in the kernels; per-row counts must fit int32
  if (p->TC * p->Hq > INT32_MAX || p->TL * p->Hkv > INT32_MAX)
    return fail(QUOKA_EUNSUPPORTED, "token totals too large");
  if ((int64_t)p->maxC * p->G > INT32_MAX) return fail(QUOKA_EUNSUPPORTED, "chunk too long");
  // the fp64 re-ranking near the selection boundaries packs positions in 24 bits
  if (p->maxC >= (1 << 24) || p->maxL >= (1 << 24))
    return fail(QUOKA_EUNSUPPORTED, "a chunk or history of 2^24 tokens or more");
  // kernels address one sequence's rows through 32-bit buffer offsets
  const int64_t elem = sh->dtype == QUOKA_BF16 ? 2 : 4;
  const int64_t row = (int64_t)p->Hkv * p->D * elem;
  if ((int64_t)p->maxL * row > INT32_MAX || (int64_t)p->maxC * row > INT32_MAX ||
      (int64_t)kv_budget * p->D * elem > INT32_MAX)
    return fail(QUOKA_EUNSUPPORTED, "a sequence's K/V rows exceed 2 GiB");
  p->q_budget = q_budget;
  p->kv_budget = kv_budget;
  p->nq_pad = (q_budget + 15) / 16 * 16;
  p->variant = QUOKA_VARIANT_QUOKA;
  return QUOKA_OK;
}

// What a baseline needs beyond make_problem's checks.
quoka_status set_variant(int32_t variant, Problem* p) {
  if (variant < QUOKA_VARIANT_QUOKA || variant > QUOKA_VARIANT_GLOBAL)
    return fail(QUOKA_EINVAL, "variant=%d is not a quoka_variant", variant);
  p->variant = variant;
  if (variant == QUOKA_VARIANT_GLOBAL && p->maxC > kQselCap)
    return fail(QUOKA_EUNSUPPORTED, "the cross-head baseline takes chunks of at most %d tokens",
                kQselCap);
  if (variant == QUOKA_VARIANT_PER_HEAD && (int64_t)p->nq_pad * p->G > kMaxHeadRows)
    return fail(QUOKA_EUNSUPPORTED,
                "the per-head baseline takes ceil(q_budget/16)*16 * H_q/H_kv <= %d rows",
                kMaxHeadRows);
  return QUOKA_OK;
}

}  // namespace

ScoreBounds score_bounds(const Problem& p) {
  const double u = 0x1p-24;
  const bool bf = p.dtype == QUOKA_BF16;
  const int GH = p.gh();
  const double nt = (bf ? 2.0 : 1.0) * p.D * GH;  // products summed per score
  // rows: g rounded to fp32 (2u, also covering the means of the one-row
  // baselines); the per-head baseline's unit rows carry an fp32 norm
  const double rows = (p.variant == QUOKA_VARIANT_PER_HEAD ? p.D / 2.0 + 3.0 : 2.0) * u;
  const double row = rows + (bf ? 0x1p-18 * 1.01 : 0.0) + 2.0 * nt * u * 1.01;
  const double eps = row + (p.D + 4.0) * u * 1.01;
  return {(float)(row * 1.001), (float)(eps * 1.001)};
}

Workspace workspace_layout(const Problem& p) {
  Workspace w;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const size_t SH = (size_t)p.S * p.Hkv;
  w.plan = take(3 * (size_t)(p.S + 1) * 4);
  w.g = take((size_t)p.TC * p.Hkv * p.D * 4);
  w.gpart = take((size_t)p.NQT * p.Hkv * p.D * 8);
  w.qcos = take((size_t)p.Hkv * p.TC * 4);
  w.qidx = take(SH * p.q_budget * 4);
  w.gsel = take(SH * p.nq_pad * p.G * p.D * 4);  // G rows per token: the per-head baseline
  w.scores = take((size_t)p.Hkv * p.TL * 4);
  w.zero_begin = o;
  w.hist = take(SH * kScoreBins * 4);
  w.chcount = take((size_t)p.Hkv * p.NKT * 4);
  // one bit per history key and head; the top-B write reads two words from
  // any key's position, up to a tile past the last key
  w.bits = take(((size_t)p.Hkv * p.TL + kTopbKeys + 64) / 32 * 4);
  w.zero_end = o;
  w.thr = take(SH * sizeof(Threshold));
  w.cand = take((size_t)p.Hkv * p.TL * 8);
  w.ctcount = take((size_t)p.Hkv * p.NKT * 4);
  w.qkey = take((size_t)p.Hkv * p.TC * 8);
  w.row0 = take(SH * p.D * 8);
  w.gtcount = take((size_t)p.Hkv * p.NKT * 4);
  w.select_end = o;
  w.selidx = take(SH * p.kv_budget * 4);
  // the attention runs after the selection: its partial states reuse the
  // selection's scratch when they fit there (never the kept indices)
  const size_t attn = attn_workspace_bytes(p);
  w.attn = attn <= w.select_end ? 0 : take(attn);
  w.total = o;
  return w;
}

}  // namespace quoka

using namespace quoka;

namespace {

// events, when given: four events recorded before the query side, after it,
// after the scorer and after the top-B launches.
quoka_status run_select(const Problem& p, const Workspace& w, const void* q, const void* k_hist,
                        int32_t* sel_idx, int32_t* q_idx_opt, float* qcos_opt, float* scores_opt,
                        char* ws, hipStream_t st, hipEvent_t* events = nullptr) {
  quoka_status rc = ensure_lds(p);
  if (rc != QUOKA_OK) return rc;
  float* qcos = qcos_opt ? qcos_opt : (float*)(ws + w.qcos);
  float* scores = scores_opt ? scores_opt : (float*)(ws + w.scores);
  int32_t* qidx = q_idx_opt ? q_idx_opt : (int32_t*)(ws + w.qidx);
  auto mark = [&](int i) -> quoka_status {
    return events ? hip_check(hipEventRecord(events[i], st), "hipEventRecord", st) : QUOKA_OK;
  };
  if ((rc = mark(0))) return rc;
  if ((rc = hip_check(launch_qprep(p, q, ws, w, qcos, qcos_opt != nullptr, qidx, sel_idx, st), "qprep", st)))
    return rc;
  if ((rc = mark(1))) return rc;
  if ((rc = hip_check(launch_scorer(p, k_hist, ws, w, scores, st), "scorer", st))) return rc;
  if ((rc = mark(2))) return rc;
  if ((rc = hip_check(launch_topb(p, q, k_hist, qidx, ws, w, scores, sel_idx, st), "topb", st)))
    return rc;
  if ((rc = mark(3))) return rc;
  if (debug_mode()) {
    const DebugItem it{sel_idx, n_sel(p), kDebugIdxSelection, kDbgSelOut};
    return debug_run(p, &it, 1, st);
  }
  return QUOKA_OK;
}

#define QUOKA_NEED(ptr, total)                                                          \
  do {                                                                                  \
    if (!(ptr) && (total) > 0) return fail(QUOKA_EINVAL, "%s is null", #ptr);           \
    if ((ptr) && !aligned16(ptr)) return fail(QUOKA_EINVAL, "%s is not 16-byte aligned", #ptr); \
  } while (0)

// Scratch of quoka_prefill_chunk_static: one array per device the library
// runs on, held until the process ends. Host code never uses its name as an
// address: the device address comes from hipGetSymbolAddress, per device.
constexpr size_t kStaticScratchBytes = (size_t)QUOKA_STATIC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kStaticScratchBytes];

quoka_status static_scratch(char** out) {
  static std::mutex mu;
  static char* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(QUOKA_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(QUOKA_EUNSUPPORTED, "device ordinal %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(QUOKA_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    addr[dev] = (char*)ptr;
  }
  *out = addr[dev];
  return QUOKA_OK;
}

// The attention entry points' workspace: needed only when the shape splits
// its keys (attn_workspace_bytes > 0).
quoka_status attn_ws_check(const Problem& p, const void* ws, size_t ws_bytes) {
  const size_t need = attn_workspace_bytes(p);
  if (need == 0) return QUOKA_OK;
  if (!ws) return fail(QUOKA_EWORKSPACE, "this shape needs %zu bytes of workspace, none given", need);
  if (!aligned16(ws)) return fail(QUOKA_EINVAL, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(QUOKA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  return QUOKA_OK;
}

}  // namespace

extern "C" {

quoka_status quoka_workspace_bytes(const quoka_shape* shape, int32_t q_budget,
                                   int32_t kv_budget, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(QUOKA_EINVAL, "bytes is null");
  Problem p;
  quoka_status rc = make_problem(shape, q_budget, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  *bytes = workspace_layout(p).total;
  return QUOKA_OK;
}

quoka_status quoka_select(const quoka_shape* shape, const void* q, const void* k_hist,
                          int32_t q_budget, int32_t kv_budget, int32_t* sel_idx,
                          int32_t* q_idx_opt, float* qcos_opt, float* scores_opt, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, q_budget, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(sel_idx, 1);
  if (!ws) return fail(QUOKA_EWORKSPACE, "workspace is null");
  if (!aligned16(ws)) return fail(QUOKA_EINVAL, "workspace is not 16-byte aligned");
  const Workspace w = workspace_layout(p);
  if (ws_bytes < w.total)
    return fail(QUOKA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_hist, n_hist(p), kDebugRowsAll, kDbgKHist}}, stream)))
    return rc;
  return run_select(p, w, q, k_hist, sel_idx, q_idx_opt, qcos_opt, scores_opt, (char*)ws,
                    stream);
}

quoka_status quoka_select_profiled(const quoka_shape* shape, const void* q, const void* k_hist,
                                   int32_t q_budget, int32_t kv_budget, int32_t* sel_idx,
                                   void* ws, size_t ws_bytes, hipEvent_t* events,
                                   hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, q_budget, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(sel_idx, 1);
  if (!events) return fail(QUOKA_EINVAL, "events is null");
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return fail(QUOKA_EINVAL, "events[%d] is null", i);
  if (!ws) return fail(QUOKA_EWORKSPACE, "workspace is null");
  if (!aligned16(ws)) return fail(QUOKA_EINVAL, "workspace is not 16-byte aligned");
  const Workspace w = workspace_layout(p);
  if (ws_bytes < w.total)
    return fail(QUOKA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_hist, n_hist(p), kDebugRowsAll, kDbgKHist}}, stream)))
    return rc;
  return run_select(p, w, q, k_hist, sel_idx, nullptr, nullptr, nullptr, (char*)ws, stream,
                    events);
}

quoka_status quoka_select_variant(const quoka_shape* shape, int32_t variant, const void* q,
                                  const void* k_hist, int32_t q_budget, int32_t kv_budget,
                                  int32_t* sel_idx, int32_t* q_idx_opt, float* qcos_opt,
                                  float* scores_opt, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, q_budget, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  if ((rc = set_variant(variant, &p)) != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(sel_idx, 1);
  if (!ws) return fail(QUOKA_EWORKSPACE, "workspace is null");
  if (!aligned16(ws)) return fail(QUOKA_EINVAL, "workspace is not 16-byte aligned");
  const Workspace w = workspace_layout(p);
  if (ws_bytes < w.total)
    return fail(QUOKA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_hist, n_hist(p), kDebugRowsAll, kDbgKHist}}, stream)))
    return rc;
  return run_select(p, w, q, k_hist, sel_idx, q_idx_opt, qcos_opt, scores_opt, (char*)ws,
                    stream);
}

quoka_status quoka_gather(const quoka_shape* shape, const void* k_hist, const void* v_hist,
                          const int32_t* sel_idx, int32_t kv_budget, void* k_sel, void* v_sel,
                          hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, 1, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(v_hist, p.TL);
  QUOKA_NEED(sel_idx, 1);
  QUOKA_NEED(k_sel, 1);
  QUOKA_NEED(v_sel, 1);
  if ((rc = debug_inputs(p, {{k_hist, n_hist(p), kDebugRowsAll, kDbgKHist},
                             {v_hist, n_hist(p), kDebugRowsAll, kDbgVHist},
                             {sel_idx, n_sel(p), kDebugIdxInput, kDbgSelIn}}, stream)))
    return rc;
  return hip_check(launch_gather(p, k_hist, v_hist, sel_idx, k_sel, v_sel, stream), "gather",
                   stream);
}

quoka_status quoka_check_selection(const quoka_shape* shape, const int32_t* sel_idx,
                                   int32_t kv_budget, hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, 1, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(sel_idx, 1);
  const DebugItem it{sel_idx, n_sel(p), kDebugIdxSelection, kDbgSelOut};
  return debug_run(p, &it, 1, stream);
}

quoka_status quoka_attn_plan(const quoka_shape* shape, int32_t kv_budget, int32_t* kernel,
                             int32_t* key_ranges) {
  g_err[0] = 0;
  if (!kernel || !key_ranges) return fail(QUOKA_EINVAL, "kernel or key_ranges is null");
  Problem p;
  quoka_status rc = make_problem(shape, 1, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  int k = 0, n = 1;
  attn_describe(p, &k, &n);
  *kernel = k;
  *key_ranges = n;
  return QUOKA_OK;
}

quoka_status quoka_attn_workspace_bytes(const quoka_shape* shape, int32_t kv_budget,
                                        size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(QUOKA_EINVAL, "bytes is null");
  Problem p;
  quoka_status rc = make_problem(shape, 1, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  *bytes = attn_workspace_bytes(p);
  return QUOKA_OK;
}

quoka_status quoka_chunk_attn(const quoka_shape* shape, const void* q, const void* k_sel,
                              const void* v_sel, int32_t kv_budget, const void* k_chunk,
                              const void* v_chunk, float softmax_scale, void* out, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, 1, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_sel, 1);
  QUOKA_NEED(v_sel, 1);
  QUOKA_NEED(k_chunk, p.TC);
  QUOKA_NEED(v_chunk, p.TC);
  QUOKA_NEED(out, p.TC);
  if (!std::isfinite(softmax_scale)) return fail(QUOKA_EINVAL, "softmax_scale is not finite");
  if ((rc = attn_ws_check(p, ws, ws_bytes))) return rc;
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_sel, n_sel(p) * p.D, kDebugRowsSel, kDbgKSel},
                             {v_sel, n_sel(p) * p.D, kDebugRowsSel, kDbgVSel},
                             {k_chunk, n_chunk(p), kDebugRowsAll, kDbgKChunk},
                             {v_chunk, n_chunk(p), kDebugRowsAll, kDbgVChunk}}, stream)))
    return rc;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.D);
  return hip_check(
      launch_attention(p, q, k_sel, v_sel, nullptr, k_chunk, v_chunk, scale, out, ws, stream),
      "attention", stream);
}

quoka_status quoka_chunk_attn_gather(const quoka_shape* shape, const void* q, const void* k_hist,
                                     const void* v_hist, const int32_t* sel_idx,
                                     int32_t kv_budget, const void* k_chunk, const void* v_chunk,
                                     float softmax_scale, void* out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, 1, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(v_hist, p.TL);
  QUOKA_NEED(sel_idx, 1);
  QUOKA_NEED(k_chunk, p.TC);
  QUOKA_NEED(v_chunk, p.TC);
  QUOKA_NEED(out, p.TC);
  if (!std::isfinite(softmax_scale)) return fail(QUOKA_EINVAL, "softmax_scale is not finite");
  if ((rc = attn_ws_check(p, ws, ws_bytes))) return rc;
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_hist, n_hist(p), kDebugRowsAll, kDbgKHist},
                             {v_hist, n_hist(p), kDebugRowsAll, kDbgVHist},
                             {sel_idx, n_sel(p), kDebugIdxInput, kDbgSelIn},
                             {k_chunk, n_chunk(p), kDebugRowsAll, kDbgKChunk},
                             {v_chunk, n_chunk(p), kDebugRowsAll, kDbgVChunk}}, stream)))
    return rc;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.D);
  return hip_check(
      launch_attention(p, q, k_hist, v_hist, sel_idx, k_chunk, v_chunk, scale, out, ws, stream),
      "attention", stream);
}

quoka_status quoka_prefill_chunk(const quoka_shape* shape, const void* q, const void* k_hist,
                                 const void* v_hist, const void* k_chunk, const void* v_chunk,
                                 int32_t q_budget, int32_t kv_budget, float softmax_scale,
                                 void* out, int32_t* sel_idx_opt, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, q_budget, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(v_hist, p.TL);
  QUOKA_NEED(k_chunk, p.TC);
  QUOKA_NEED(v_chunk, p.TC);
  QUOKA_NEED(out, p.TC);
  if (!std::isfinite(softmax_scale)) return fail(QUOKA_EINVAL, "softmax_scale is not finite");
  if (!ws) return fail(QUOKA_EWORKSPACE, "workspace is null");
  if (!aligned16(ws)) return fail(QUOKA_EINVAL, "workspace is not 16-byte aligned");
  const Workspace w = workspace_layout(p);
  if (ws_bytes < w.total)
    return fail(QUOKA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  char* base = (char*)ws;
  int32_t* sel = sel_idx_opt ? sel_idx_opt : (int32_t*)(base + w.selidx);
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_hist, n_hist(p), kDebugRowsAll, kDbgKHist},
                             {v_hist, n_hist(p), kDebugRowsAll, kDbgVHist},
                             {k_chunk, n_chunk(p), kDebugRowsAll, kDbgKChunk},
                             {v_chunk, n_chunk(p), kDebugRowsAll, kDbgVChunk}}, stream)))
    return rc;
  rc = run_select(p, w, q, k_hist, sel, nullptr, nullptr, nullptr, base, stream);
  if (rc != QUOKA_OK) return rc;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.D);
  return hip_check(launch_attention(p, q, k_hist, v_hist, sel, k_chunk, v_chunk, scale, out,
                                   base + w.attn, stream),
                   "attention", stream);
}

quoka_status quoka_prefill_chunk_static(const quoka_shape* shape, const void* q,
                                        const void* k_hist, const void* v_hist,
                                        const void* k_chunk, const void* v_chunk,
                                        int32_t q_budget, int32_t kv_budget,
                                        float softmax_scale, void* out, int32_t* sel_idx_opt,
                                        hipStream_t stream) {
  g_err[0] = 0;
  Problem p;
  quoka_status rc = make_problem(shape, q_budget, kv_budget, &p);
  if (rc != QUOKA_OK) return rc;
  QUOKA_NEED(q, p.TC);
  QUOKA_NEED(k_hist, p.TL);
  QUOKA_NEED(v_hist, p.TL);
  QUOKA_NEED(k_chunk, p.TC);
  QUOKA_NEED(v_chunk, p.TC);
  QUOKA_NEED(out, p.TC);
  if (!std::isfinite(softmax_scale)) return fail(QUOKA_EINVAL, "softmax_scale is not finite");
  const Workspace w = workspace_layout(p);
  if (w.total > kStaticScratchBytes)
    return fail(QUOKA_EUNSUPPORTED,
                "this problem needs %zu bytes of scratch; the static scratch holds %zu "
                "(use quoka_prefill_chunk with a workspace)",
                w.total, kStaticScratchBytes);
  char* base = nullptr;
  if ((rc = static_scratch(&base))) return rc;
  int32_t* sel = sel_idx_opt ? sel_idx_opt : (int32_t*)(base + w.selidx);
  if ((rc = debug_inputs(p, {{q, n_q(p), kDebugRowsAll, kDbgQ},
                             {k_hist, n_hist(p), kDebugRowsAll, kDbgKHist},
                             {v_hist, n_hist(p), kDebugRowsAll, kDbgVHist},
                             {k_chunk, n_chunk(p), kDebugRowsAll, kDbgKChunk},
                             {v_chunk, n_chunk(p), kDebugRowsAll, kDbgVChunk}}, stream)))
    return rc;
  rc = run_select(p, w, q, k_hist, sel, nullptr, nullptr, nullptr, base, stream);
  if (rc != QUOKA_OK) return rc;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.D);
  return hip_check(launch_attention(p, q, k_hist, v_hist, sel, k_chunk, v_chunk, scale, out,
                                   base + w.attn, stream),
                   "attention", stream);
}

}  // extern "C"

namespace {

// The workspace of a prompt: per-chunk offsets, one chunk's kept indices,
// then the per-chunk workspace of the largest chunk problem (reused by every
// chunk in stream order).
struct PromptLayout {
  int nch;
  size_t cu, sel, chunk_ws, chunk_ws_bytes, total;
};

quoka_status prompt_layout(const quoka_prompt* pr, int32_t q_budget, int32_t kv_budget,
                           PromptLayout* lay) {
  if (!pr) return fail(QUOKA_EINVAL, "prompt is null");
  if (pr->prompt_len < 1) return fail(QUOKA_EINVAL, "prompt_len=%d must be >= 1", pr->prompt_len);
  if (pr->chunk_len < 1) return fail(QUOKA_EINVAL, "chunk_len=%d must be >= 1", pr->chunk_len);
  const int T = pr->prompt_len, Bc = pr->chunk_len;
  lay->nch = (int)(((int64_t)T + Bc - 1) / Bc);
  size_t need = 0;
  for (int i = 0; i < lay->nch; ++i) {
    const int32_t a = (int32_t)std::min<int64_t>((int64_t)i * Bc, T);
    const int32_t b = (int32_t)std::min<int64_t>((int64_t)a + Bc, T);
    const int32_t cc[2] = {0, b - a}, ch[2] = {0, a};
    // sizing only: the device offsets are not read (the host arrays stand in)
    const quoka_shape sh = {1, pr->num_q_heads, pr->num_kv_heads, pr->head_dim, pr->dtype,
                            cc, ch, cc, ch};
    Problem p;
    const quoka_status rc = make_problem(&sh, q_budget, kv_budget, &p);
    if (rc != QUOKA_OK) return rc;
    need = std::max(need, workspace_layout(p).total);
  }
  size_t o = 0;
  lay->cu = o;
  o = align_up(o + (size_t)lay->nch * 4 * sizeof(int32_t), 256);
  lay->sel = o;
  o = align_up(o + (size_t)pr->num_kv_heads * kv_budget * sizeof(int32_t), 256);
  lay->chunk_ws = o;
  lay->chunk_ws_bytes = need;
  lay->total = o + need;
  return QUOKA_OK;
}

}  // namespace

extern "C" {

quoka_status quoka_prompt_workspace_bytes(const quoka_prompt* prompt, int32_t q_budget,
                                          int32_t kv_budget, size_t* bytes) {
  g_err[0] = 0;
  if (!bytes) return fail(QUOKA_EINVAL, "bytes is null");
  PromptLayout lay;
  const quoka_status rc = prompt_layout(prompt, q_budget, kv_budget, &lay);
  if (rc != QUOKA_OK) return rc;
  *bytes = lay.total;
  return QUOKA_OK;
}

quoka_status quoka_prefill_prompt(const quoka_prompt* prompt, const void* q, const void* k,
                                  const void* v, int32_t q_budget, int32_t kv_budget,
                                  float softmax_scale, void* out, int32_t* sel_idx_opt,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  g_err[0] = 0;
  PromptLayout lay;
  quoka_status rc = prompt_layout(prompt, q_budget, kv_budget, &lay);
  if (rc != QUOKA_OK) return rc;
  const int T = prompt->prompt_len, Bc = prompt->chunk_len;
  QUOKA_NEED(q, T);
  QUOKA_NEED(k, T);
  QUOKA_NEED(v, T);
  QUOKA_NEED(out, T);
  QUOKA_NEED(sel_idx_opt, 0);
  if (!std::isfinite(softmax_scale)) return fail(QUOKA_EINVAL, "softmax_scale is not finite");
  if (!ws) return fail(QUOKA_EWORKSPACE, "workspace is null");
  if (!aligned16(ws)) return fail(QUOKA_EINVAL, "workspace is not 16-byte aligned");
  if (ws_bytes < lay.total)
    return fail(QUOKA_EWORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, lay.total);
  char* base = (char*)ws;
  int32_t* cu = (int32_t*)(base + lay.cu);
  if ((rc = hip_check(launch_prompt_offsets(T, Bc, lay.nch, cu, stream), "prompt offsets",
                      stream)))
    return rc;
  const size_t elem = prompt->dtype == QUOKA_BF16 ? 2 : 4;
  const size_t qrow = (size_t)prompt->num_q_heads * prompt->head_dim * elem;
  const size_t krow = (size_t)prompt->num_kv_heads * prompt->head_dim * elem;
  const size_t sel_chunk = (size_t)prompt->num_kv_heads * kv_budget;
  for (int i = 0; i < lay.nch; ++i) {
    const int32_t a = i * Bc, b = (int32_t)std::min<int64_t>((int64_t)a + Bc, T);
    const int32_t cc[2] = {0, b - a}, ch[2] = {0, a};
    const quoka_shape sh = {1, prompt->num_q_heads, prompt->num_kv_heads, prompt->head_dim,
                            prompt->dtype, cu + 4 * i, cu + 4 * i + 2, cc, ch};
    Problem p;
    if ((rc = make_problem(&sh, q_budget, kv_budget, &p))) return rc;
    const Workspace w = workspace_layout(p);
    int32_t* sel = sel_idx_opt ? sel_idx_opt + (size_t)i * sel_chunk : (int32_t*)(base + lay.sel);
    if (debug_mode()) {
      // the whole prompt's rows once, then every chunk's device offsets
      const int64_t nq = (int64_t)T * p.Hq * p.D, nk = (int64_t)T * p.Hkv * p.D;
      if (i == 0 && (rc = debug_inputs(p, {{q, nq, kDebugRowsAll, kDbgQ},
                                           {k, nk, kDebugRowsAll, kDbgK},
                                           {v, nk, kDebugRowsAll, kDbgV}}, stream)))
        return rc;
      if ((rc = debug_offsets(p))) return rc;
    }
    const char* qi = (const char*)q + (size_t)a * qrow;
    rc = run_select(p, w, qi, k, sel, nullptr, nullptr, nullptr, base + lay.chunk_ws, stream);
    if (rc != QUOKA_OK) return rc;
    const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)p.D);
    if ((rc = hip_check(launch_attention(p, qi, k, v, sel, (const char*)k + (size_t)a * krow,
                                         (const char*)v + (size_t)a * krow, scale,
                                         (char*)out + (size_t)a * qrow,
                                         base + lay.chunk_ws + w.attn, stream),
                        "attention", stream)))
      return rc;
  }
  return QUOKA_OK;
}

const char* quoka_strerror(quoka_status status) {
  switch (status) {
    case QUOKA_OK: return "success";
    case QUOKA_EINVAL: return "invalid argument";
    case QUOKA_EUNSUPPORTED: return "unsupported configuration";
    case QUOKA_EWORKSPACE: return "workspace missing or too small";
    case QUOKA_EHIP: return "HIP error";
    case QUOKA_ECHECK: return "result failed its check";
  }
  return "unknown status";
}

const char* quoka_last_error(void) { return g_err; }

}  // extern "C"
