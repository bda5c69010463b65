// Host-side plumbing shared by the launchers and the C ABI: the workspace
// layout, the per-call problem description and the launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "quoka.h"

namespace quoka {

// Tilings (all per sequence; tiles never straddle two sequences).
constexpr int kQprepTokens = 64;     // tokens per query-prep workgroup, at most
constexpr int kQprepWavesTotal = 16; // waves per query-prep workgroup
constexpr int kScoreKeysMin = 256;   // history keys per scorer workgroup: one block per wave...
constexpr int kScoreKeysMax = 2048;  // ...up to eight blocks per wave, streamed
constexpr int kScoreMaxBlocks = 512; // one round of scorer workgroups (two per CU)
constexpr int kTopbKeys = 2048;      // history keys per top-B workgroup
constexpr int kCandCap = 6144;       // candidates the top-B refinement keeps in LDS
constexpr int kQselCap = 12288;      // chunk tokens whose cosines the query select stages in LDS

// How the scorer forms a key's score from the rows the query select lays out.
enum ScoreMode {
  kModeCos = 0,    // max over rows of g . k / |k| (QUOKA and the cosine baselines)
  kModeDot = 1,    // max over rows of g . k, unbounded (histogram by score_bin_raw)
  kModeHeads = 2,  // rows hold each head separately: max over tokens of mean over heads
};

struct Problem {
  int S, Hq, Hkv, G, D;
  quoka_dtype dtype;
  const int32_t* cu_chunk;   // device
  const int32_t* cu_hist;    // device
  const int32_t* cu_chunk_h; // host
  const int32_t* cu_hist_h;  // host
  int64_t TC, TL;            // total chunk tokens, total history keys
  int64_t NQT, NSB, NKT;     // total qprep / scorer / top-B tiles over sequences
  int qtok;                  // tokens per query-prep tile: 64, 32 or 16
  int maxC, maxL;            // longest chunk, longest history
  int q_budget, kv_budget, nq_pad;
  int score_keys;            // history keys per scorer workgroup (a power of two, 256..2048)
  int variant;               // quoka_variant
  int mode() const {
    return variant == QUOKA_VARIANT_DOT ? kModeDot
         : variant == QUOKA_VARIANT_PER_HEAD ? kModeHeads : kModeCos;
  }
  // the scorer reads one row per (sequence, head): the mean-query baselines
  bool one_row() const {
    return variant == QUOKA_VARIANT_MEAN_QUERIES || variant == QUOKA_VARIANT_MEAN_QUERY;
  }
  int gh() const { return variant == QUOKA_VARIANT_PER_HEAD ? G : 1; }  // rows per kept token
};

// Largest (kept rows) x (heads) the per-head baseline lays out (LDS-bound).
constexpr int kMaxHeadRows = 640;

// Byte offsets of the workspace regions (each 256-byte aligned).
struct Workspace {
  size_t plan;      // int32 qt_off[S+1], sb_off[S+1], kt_off[S+1]
  size_t g;         // float [TC, Hkv, D]  pre-aggregated queries
  size_t gpart;     // double [NQT, Hkv, D] per-tile sums of g
  size_t qcos;      // float [Hkv, TC]
  size_t qidx;      // int32 [S, Hkv, q_budget]
  size_t gsel;      // 4 B x [S, Hkv, nq_pad, G, D]  kept queries laid out for the scorer
  size_t scores;    // float [Hkv, TL]
  size_t hist;      // uint32 [S, Hkv, kScoreBins]
  size_t thr;       // Threshold [S, Hkv]
  size_t ctcount;   // uint32 [Hkv, NKT] candidates per tile
  size_t cand;      // uint64 [Hkv, TL] candidates, each tile's in its own key range
  size_t gtcount;   // uint32 [Hkv, NKT] keys above the threshold bin per tile
  size_t chcount;   // uint32 [Hkv, NKT] chosen candidates per tile
  size_t bits;      // uint32 bitmap over [Hkv, TL]: chosen candidates
  size_t qkey;      // uint64 [Hkv, TC] tokens re-ranked in fp64
  size_t row0;      // double [S, Hkv, D] the one-row baselines' row in fp64
  size_t selidx;    // int32 [S, Hkv, B]  (prefill path)
  size_t attn;      // the attention's partial states (after the selection;
                    // over its scratch when they fit there)
  size_t select_end, total;
  size_t zero_begin, zero_end;  // [hist .. chcount] region cleared per call
};

struct Threshold {
  int32_t bstar;           // bin holding the B_eff-th score; -1 = keep everything
  int32_t pad;
  double lo, hi;           // candidates: scores in [lo, hi]; above hi kept, below lo not
};

// |fp32 cosine to the mean query - fp64 cosine|. The stored g is the fp64
// mean of unit head rows rounded once to fp32 (relative error 2^-24 per
// element, so the cosine moves by at most 2^-24); the fp64 products with the
// fp64 mean query add ~1e-13 and the quotient's rounding to fp32 2^-24: 2^-23
// with a factor of two to spare.
constexpr float kQcosErr = 0x1p-22f;

// Error bounds of the scorer's fp32 values against the fp64 definition:
//   eps_row bounds |fp32 product - fp64 product| of one kept row with a key,
//           in units of |k| (rows have norm <= 1): the row's own rounding to
//           fp32, the hi/lo bf16 split (residual <= 2^-18 |g| per element)
//           and the fp32 accumulation of nt products (at most nt roundings,
//           each <= 2^-23 relative to the running sum whether the adder
//           rounds to nearest or toward zero);
//   eps     bounds |fp32 score - fp64 score|: eps_row plus |k| from a sum of
//           d squares, its square root and the quotient.
struct ScoreBounds {
  float eps_row, eps;
};
ScoreBounds score_bounds(const Problem& p);

Workspace workspace_layout(const Problem& p);

// Records the message quoka_last_error() returns on this thread; returns st.
quoka_status fail(quoka_status st, const char* fmt, ...);

// Launchers (enqueue only; return hipGetLastError()).
// Raise the dynamic-LDS limit of the scorer kernels (they hold the kept
// queries and a score histogram on chip).
// bytes_heads is for the per-head baseline's kernels.
hipError_t set_scorer_lds_limit(int bytes, int bytes_heads);

// Plan and counter clearing, query prep, cosines and the lowest-cosine
// select; also writes the -1 padding of sel_idx past each problem's B_eff.
// want_cos: the caller asked for the cosines (else they are computed only when
// some chunk has more tokens than q_budget, i.e. when the subselection needs them).
hipError_t launch_qprep(const Problem& p, const void* q, char* ws, const Workspace& w,
                        float* qcos, bool want_cos, int32_t* qidx, int32_t* sel_idx,
                        hipStream_t st);
size_t scorer_lds_bytes(const Problem& p);
hipError_t launch_scorer(const Problem& p, const void* k_hist, char* ws, const Workspace& w,
                         float* scores, hipStream_t st);
hipError_t launch_topb(const Problem& p, const void* q, const void* k_hist, const int32_t* qidx,
                       char* ws, const Workspace& w, const float* scores, int32_t* sel_idx,
                       hipStream_t st);
hipError_t launch_gather(const Problem& p, const void* k_hist, const void* v_hist,
                         const int32_t* sel_idx, void* k_sel, void* v_sel, hipStream_t st);
// sel == nullptr: history rows are k_sel / v_sel [S, Hkv, kv_budget, D];
// otherwise k_sel / v_sel are k_hist / v_hist and row b of (s, h) is history
// row sel[s, h, b] (gather fused into the attention).
// Shapes that fill at most half the chip split each row tile's keys into
// ranges whose partial softmax states (fp32 O, max, sum per row and range) go
// to attn_ws, attn_workspace_bytes(p) bytes (0: no split, attn_ws unused),
// and are merged by a second launch.
size_t attn_workspace_bytes(const Problem& p);
// The attention kernel (quoka_attn_kernel) and key ranges launch_attention uses.
void attn_describe(const Problem& p, int* kernel, int* key_ranges);
hipError_t launch_attention(const Problem& p, const void* q, const void* k_sel,
                            const void* v_sel, const int32_t* sel, const void* k_chunk,
                            const void* v_chunk, float scale, void* out, void* attn_ws,
                            hipStream_t st);

// Per-chunk offsets {0, C_i, 0, L_i} of a one-sequence prompt split in chunks.
hipError_t launch_prompt_offsets(int T, int chunk_len, int nch, int32_t* cu, hipStream_t st);

}  // namespace quoka
