/*
 * quoka.h - C ABI of the QUOKA per-chunk hot path on MI355X (gfx950).
 *
 * QUOKA ("QUOKA: Query-Oriented KV Selection For Efficient LLM Prefill")
 * speeds up chunked prefill by letting each chunk attend to a small subset of
 * the cached history. Per (sequence, KV head) the library
 *   1. reduces the chunk's queries of the KV head's query heads to a mean
 *      query and keeps the N_q queries least similar to it;
 *   2. scores every history key by cosine similarity against the kept
 *      queries, taking the max over kept tokens of the mean over the group's
 *      heads, and keeps the top-B keys;
 *   3. gathers the kept keys' K/V rows;
 *   4. runs softmax attention of every chunk query (original heads) over the
 *      kept history plus the chunk's own keys under a causal mask.
 * Sources: the QUOKA paper summary (hw-hk.tistory.com/367), sections "QUOKA
 * Method" and "Background > Chunked prefill", and "QUOKA Explained: Choosing
 * Which KV History Attention Should Read" (reactapp.top).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers unless their name ends in _host. The caller
 * owns every buffer; the library never allocates or frees memory and keeps no
 * state between calls except a per-device cache of device properties, so calls
 * on different streams may run concurrently as long as they share no output
 * or workspace buffer.
 *
 * Layouts are token-major and contiguous (elements of `dtype`):
 *   q                [sum_s C_s, H_q,  d]   chunk queries
 *   k_hist, v_hist   [sum_s L_s, H_kv, d]   cached history K/V (never modified)
 *   k_chunk, v_chunk [sum_s C_s, H_kv, d]   the chunk's own K/V
 *   out              [sum_s C_s, H_q,  d]
 *   k_sel, v_sel     [S, H_kv, B, d]        gathered rows
 *   sel_idx          [S, H_kv, B]   int32   kept history positions (0-based
 *                                           within the sequence), ascending,
 *                                           -1 padding past B_eff
 * Query head j belongs to KV head j / (H_q / H_kv) (contiguous GQA groups).
 * Per sequence the budgets are clamped to the data:
 *   N_q,eff = min(q_budget, C_s), B_eff = min(kv_budget, L_s).
 * Ties in either selection go to the lower token / key index, so every result
 * is unique. Inputs must be finite.
 *
 * Errors: validation runs on the host before anything is enqueued and returns
 * QUOKA_EINVAL / QUOKA_EUNSUPPORTED / QUOKA_EWORKSPACE without touching the
 * GPU; quoka_last_error() then names the offending argument. A failed launch
 * returns QUOKA_EHIP. Device faults surface asynchronously, as with any HIP
 * call; set the environment variable QUOKA_SYNC=1 to synchronize the stream
 * after every launch and report them as QUOKA_EHIP.
 *
 * Debug mode: with the environment variable QUOKA_DEBUG set (to anything but
 * "0"; read on every call) each entry point also checks on the device, before
 * its first compute kernel, what the host cannot see, and synchronizes the
 * stream after every launch:
 *   - the device offset arrays hold the host copies' values;
 *   - every element of q, k_hist, v_hist, k_chunk, v_chunk it reads is finite
 *     (k_sel / v_sel: the rows below B_eff, the only ones read);
 *   - a sel_idx it takes as input holds -1 or positions in [0, L_s) (stricter
 *     than quoka_chunk_attn_gather's own contract, which reads any other value
 *     as a zero row: in debug mode such a value is reported);
 * any of these fails with QUOKA_EINVAL and a message naming the argument and
 * the first offending element. A sel_idx the call writes is then checked as
 * quoka_check_selection does (QUOKA_ECHECK). The checks scan every input, so
 * debug mode is for finding a caller's or the library's mistake, not for
 * timing; calls in debug mode on one device are serialized.
 */
#ifndef QUOKA_H
#define QUOKA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum quoka_status {
  QUOKA_OK = 0,
  QUOKA_EINVAL = 1,        /* a null pointer, negative size or inconsistent offsets */
  QUOKA_EUNSUPPORTED = 2,  /* well-formed but outside what is built (head_dim, budget) */
  QUOKA_EWORKSPACE = 3,    /* workspace null or smaller than quoka_workspace_bytes() */
  QUOKA_EHIP = 4,          /* a HIP launch or query failed */
  QUOKA_ECHECK = 5         /* a result failed its check (QUOKA_DEBUG mode,
                              quoka_check_selection) */
} quoka_status;

typedef enum quoka_dtype {
  QUOKA_F32 = 0,           /* fp32 everywhere, VALU kernels */
  QUOKA_BF16 = 1           /* bf16 Q/K/V/out; fp32 arithmetic; MFMA kernels */
} quoka_dtype;

/* Problem shape. head_dim must be 64 or 128; num_q_heads a multiple of
 * num_kv_heads. cu_chunk / cu_hist are prefix offsets of the chunk and
 * history lengths ([0] == 0, non-decreasing). The device and host copies must
 * hold the same values: the host copy sizes the launch grids, the kernels read
 * the device copy. */
typedef struct quoka_shape {
  int32_t num_seqs;               /* S >= 1 */
  int32_t num_q_heads;            /* H_q */
  int32_t num_kv_heads;           /* H_kv */
  int32_t head_dim;               /* d */
  quoka_dtype dtype;
  const int32_t* cu_chunk;        /* device [S + 1] */
  const int32_t* cu_hist;         /* device [S + 1] */
  const int32_t* cu_chunk_host;   /* host   [S + 1] */
  const int32_t* cu_hist_host;    /* host   [S + 1] */
} quoka_shape;

/* Largest q_budget the scorer holds on chip (kept queries per KV head). */
#define QUOKA_MAX_Q_BUDGET 128

/* Bytes of device workspace quoka_select / quoka_prefill_chunk need for this
 * shape and these budgets (written to *bytes); they include the attention's
 * partial states (quoka_attn_workspace_bytes), which quoka_prefill_chunk keeps
 * there, so the same workspace also serves quoka_chunk_attn(_gather). */
quoka_status quoka_workspace_bytes(const quoka_shape* shape, int32_t q_budget,
                                   int32_t kv_budget, size_t* bytes);

/* Selection: steps 1 and 2 above ("QUOKA Method": query subselection,
 * cosine scoring, aggregation across queries and KV groups; "QUOKA Explained":
 * "Pick the queries that disagree with the crowd" through "From scores to a
 * smaller KV set").
 *   q, k_hist    inputs (dtype of shape)
 *   q_budget     N_q, 1 .. QUOKA_MAX_Q_BUDGET
 *   kv_budget    B >= 1
 *   sel_idx      out [S, H_kv, kv_budget] int32
 *   q_idx_opt    optional out [S, H_kv, q_budget] int32: kept chunk tokens,
 *                ascending, -1 padding
 *   qcos_opt     optional out [H_kv, sum C] float: each token's cosine to its
 *                chunk's mean query
 *   scores_opt   optional out [H_kv, sum L] float: each history key's score
 *   ws, ws_bytes device workspace of at least quoka_workspace_bytes() bytes;
 *                its contents on entry do not matter
 */
quoka_status quoka_select(const quoka_shape* shape, const void* q,
                          const void* k_hist, int32_t q_budget,
                          int32_t kv_budget, int32_t* sel_idx,
                          int32_t* q_idx_opt, float* qcos_opt,
                          float* scores_opt, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* quoka_select (no optional outputs) with four caller-created HIP events
 * recorded on `stream`: events[0] before the query side (pre-aggregation,
 * cosines, subselection), events[1] before the key scorer, events[2] before
 * the top-B launches, events[3] after them. For measuring the stages of the
 * selection; the selection itself is the same. QUOKA_EINVAL if events or one
 * of its four entries is null. */
quoka_status quoka_select_profiled(const quoka_shape* shape, const void* q,
                                   const void* k_hist, int32_t q_budget,
                                   int32_t kv_budget, int32_t* sel_idx, void* ws,
                                   size_t ws_bytes, hipEvent_t* events,
                                   hipStream_t stream);

/* Baseline selections the pages set QUOKA against, for speed and parity
 * comparisons (the pages' accuracy claims for them need benchmark data).
 * Each replaces one step of the selection; everything else is as in
 * quoka_select. */
typedef enum quoka_variant {
  /* QUOKA itself (quoka_select). */
  QUOKA_VARIANT_QUOKA = 0,
  /* Key scores by raw dot products: s_i = max over kept tokens t of the mean
   * over the group's heads j of q_{t,j} . k_i; no normalisation ("QUOKA
   * Method > Scoring via Cosine Similarity": the scale-dependent QK^T of
   * earlier methods). The subselection still ranks by cosine. */
  QUOKA_VARIANT_DOT = 1,
  /* Mean, not max, over the kept tokens ("Aggregation Across Queries and KV
   * Groups", query axis; "QUOKA Explained", "Why take the maximum"). */
  QUOKA_VARIANT_MEAN_QUERIES = 2,
  /* No subselection: the chunk's mean query M (mean of every token's g_t)
   * scores the keys, s_i = M . k_i / |k_i| ("Background > Attention
   * Sparsity": single-query methods stretched to many queries by averaging;
   * "QUOKA Explained", "One query can choose for itself, but a chunk has
   * thousands"). q_idx_opt is all -1; qcos_opt is not written. */
  QUOKA_VARIANT_MEAN_QUERY = 3,
  /* Scores each kept token's G query heads separately against the keys and
   * averages afterwards (G times the products; "QUOKA Explained", "A wrinkle:
   * grouped-query attention"). Same scores as QUOKA up to rounding. Needs
   * 16 * ceil(q_budget / 16) * H_q / H_kv <= 640 rows and R * H_q / H_kv *
   * head_dim * 4 + 8192 bytes of LDS per workgroup (R = 16 * ceil(q_budget /
   * 16) in bf16, q_budget in fp32); QUOKA_EUNSUPPORTED beyond either limit
   * (160 KB of LDS on MI355X). */
  QUOKA_VARIANT_PER_HEAD = 4,
  /* One kept-token subset per sequence, shared by all KV heads: the N_q
   * tokens with the lowest mean over KV heads of the per-head cosines ("QUOKA
   * Explained", "A wrinkle: grouped-query attention": one selected token,
   * one query group per KV head). Scoring and top-B stay per KV head. Needs
   * every chunk to hold at most 12288 tokens (else QUOKA_EUNSUPPORTED). */
  QUOKA_VARIANT_GLOBAL = 5
} quoka_variant;

/* quoka_select with the selection of `variant` (a quoka_variant); same
 * arguments, layouts, workspace size and errors, plus QUOKA_EINVAL for an
 * unknown variant. */
quoka_status quoka_select_variant(const quoka_shape* shape, int32_t variant,
                                  const void* q, const void* k_hist,
                                  int32_t q_budget, int32_t kv_budget,
                                  int32_t* sel_idx, int32_t* q_idx_opt,
                                  float* qcos_opt, float* scores_opt, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Gather: step 3 ("QUOKA Explained", "From scores to a smaller KV set": a kept
 * key brings its value). Row b of (s, h) in k_sel / v_sel is row
 * sel_idx[s, h, b] of sequence s, head h of k_hist / v_hist; rows whose index
 * is -1 are written as zeros. Indices must be -1 or in [0, L_s). */
quoka_status quoka_gather(const quoka_shape* shape, const void* k_hist,
                          const void* v_hist, const int32_t* sel_idx,
                          int32_t kv_budget, void* k_sel, void* v_sel,
                          hipStream_t stream);

/* Checks a kept-index array against the selection's layout: for every
 * (s, h), entries b < B_eff = min(kv_budget, L_s) are strictly ascending
 * positions in [0, L_s) and entries from B_eff on are -1 (the layout every
 * quoka_select* call writes: "QUOKA Explained", "From scores to a smaller KV
 * set", the kept set is B_eff distinct history keys). Reads sel_idx
 * [S, H_kv, kv_budget] on the stream and waits for the result: QUOKA_OK, or
 * QUOKA_ECHECK with quoka_last_error() naming the first offending (s, h, b).
 * Allocates nothing; calls on one device are serialized. */
quoka_status quoka_check_selection(const quoka_shape* shape, const int32_t* sel_idx,
                                   int32_t kv_budget, hipStream_t stream);

/* Bytes of device workspace quoka_chunk_attn / quoka_chunk_attn_gather need
 * for this shape (written to *bytes). Shapes whose bf16 attention fills at
 * most half the chip (short chunks, decode steps) split each query tile's
 * keys into ranges computed by separate workgroups: softmax is shift
 * invariant, so the ranges' partial states (unnormalised O, running max, row
 * sum, fp32) combine exactly into the row's result ("Background > Chunked
 * prefill": each query attends to the kept history and its causal prefix,
 * in any order of the keys). Those states need nsplit * T_c * H_q * (4 d + 8)
 * bytes; every other shape needs 0. */
quoka_status quoka_attn_workspace_bytes(const quoka_shape* shape,
                                        int32_t kv_budget, size_t* bytes);

/* Which attention kernel quoka_chunk_attn(_gather) and quoka_prefill_chunk
 * launch for this shape, for measurement and tests (host only, nothing
 * runs): *kernel one of the quoka_attn_kernel values, *key_ranges the number
 * of key ranges each query tile's keys are split into (1: no split). */
typedef enum quoka_attn_kernel {
  QUOKA_ATTN_VALU = 0,            /* fp32: one token per lane */
  QUOKA_ATTN_ROWS32_4W = 1,       /* bf16 MFMA, 32 rows per wave, four waves */
  QUOKA_ATTN_ROWS32_8W = 2,       /* eight waves on 256 contiguous rows */
  QUOKA_ATTN_ROWS32_8W_PAIRED = 3,/* eight waves on a heavy and a light 128-row tile */
  QUOKA_ATTN_ROWS16 = 4           /* 16 rows per wave, eight waves per 128-row tile */
} quoka_attn_kernel;
quoka_status quoka_attn_plan(const quoka_shape* shape, int32_t kv_budget,
                             int32_t* kernel, int32_t* key_ranges);

/* Chunk attention: step 4 ("Background > Chunked prefill"; "QUOKA Method":
 * the reduced KV set goes to a dense attention kernel). Query row (t, j) of
 * sequence s attends to the first B_eff rows of k_sel / v_sel[s, j / G] and to
 * the chunk's keys 0..t (diagonal included).
 *   softmax_scale <= 0 selects 1 / sqrt(d).
 *   ws, ws_bytes  device workspace of at least quoka_attn_workspace_bytes()
 *                 bytes (may be null when that is 0), 16-byte aligned; its
 *                 contents on entry do not matter. Too small:
 *                 QUOKA_EWORKSPACE. */
quoka_status quoka_chunk_attn(const quoka_shape* shape, const void* q,
                              const void* k_sel, const void* v_sel,
                              int32_t kv_budget, const void* k_chunk,
                              const void* v_chunk, float softmax_scale,
                              void* out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Gather and chunk attention in one pass (the gather fused into the
 * attention: the same result as quoka_gather followed by quoka_chunk_attn,
 * without the k_sel / v_sel round trip through HBM). The kept history rows of
 * (s, h) are rows sel_idx[s, h, 0 .. B_eff) of sequence s, head h of k_hist /
 * v_hist; an index of -1 (or outside [0, L_s)) contributes a zero key and a
 * zero value, exactly as quoka_gather's zero rows would.
 *   softmax_scale <= 0 selects 1 / sqrt(d); ws, ws_bytes as for
 *   quoka_chunk_attn. */
quoka_status quoka_chunk_attn_gather(const quoka_shape* shape, const void* q,
                                     const void* k_hist, const void* v_hist,
                                     const int32_t* sel_idx, int32_t kv_budget,
                                     const void* k_chunk, const void* v_chunk,
                                     float softmax_scale, void* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* The whole hot path (select, then attention with the gather fused in) in
 * one call. sel_idx_opt, when not null, receives the kept indices as in
 * quoka_select. */
quoka_status quoka_prefill_chunk(const quoka_shape* shape, const void* q,
                                 const void* k_hist, const void* v_hist,
                                 const void* k_chunk, const void* v_chunk,
                                 int32_t q_budget, int32_t kv_budget,
                                 float softmax_scale, void* out,
                                 int32_t* sel_idx_opt, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Bytes of the device scratch quoka_prefill_chunk_static works in. */
#define QUOKA_STATIC_SCRATCH_BYTES (64u << 20)

/* quoka_prefill_chunk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, with its scratch in a static
 * device array of QUOKA_STATIC_SCRATCH_BYTES held by the library for each
 * device it runs on until the process ends (its device address is looked up
 * on the first call on a device). It allocates and frees nothing. The caller
 * still passes every input and output. Problems whose workspace
 * (quoka_workspace_bytes) exceeds that size return QUOKA_EUNSUPPORTED. Every
 * call on a device shares that device's array: calls that overlap on one
 * device (other streams or threads) race and must be ordered by the caller. */
quoka_status quoka_prefill_chunk_static(const quoka_shape* shape, const void* q,
                                        const void* k_hist, const void* v_hist,
                                        const void* k_chunk, const void* v_chunk,
                                        int32_t q_budget, int32_t kv_budget,
                                        float softmax_scale, void* out,
                                        int32_t* sel_idx_opt, hipStream_t stream);

/* A whole prompt of one sequence, processed by chunked prefill. */
typedef struct quoka_prompt {
  int32_t num_q_heads;            /* H_q */
  int32_t num_kv_heads;           /* H_kv */
  int32_t head_dim;               /* d: 64 or 128 */
  quoka_dtype dtype;
  int32_t prompt_len;             /* T >= 1 */
  int32_t chunk_len;              /* B_cp >= 1; the last chunk may be shorter */
} quoka_prompt;

/* Bytes of device workspace quoka_prefill_prompt needs (written to *bytes). */
quoka_status quoka_prompt_workspace_bytes(const quoka_prompt* prompt, int32_t q_budget,
                                          int32_t kv_budget, size_t* bytes);

/* Chunked prefill of a whole prompt with QUOKA (the paper summary's
 * "Background > Chunked prefill" and the chunked-prefill algorithm at the end
 * of "QUOKA Method"; "QUOKA Explained", "Chunked prefill"): the prompt is cut
 * into ceil(T / B_cp) chunks of B_cp tokens; chunk i runs the per-chunk path
 * (quoka_prefill_chunk) with tokens [0, i B_cp) as its history, so it keeps
 * at most kv_budget of them, and its own tokens under the causal mask. Chunk 0
 * has no history. Nothing is evicted: every chunk selects afresh from the
 * whole history.
 *   q        [T, H_q, d];  k, v [T, H_kv, d]: the keys and values the prompt
 *            writes into the cache (chunk i reads rows [0, (i+1) B_cp))
 *   out      [T, H_q, d]
 *   sel_idx_opt optional [ceil(T / B_cp), H_kv, kv_budget] int32: chunk i's
 *            kept history positions, as quoka_select writes them
 *   ws       device workspace of at least quoka_prompt_workspace_bytes(); its
 *            contents on entry do not matter
 * The chunks run in order on `stream`, one per-chunk pass each. */
quoka_status quoka_prefill_prompt(const quoka_prompt* prompt, const void* q, const void* k,
                                  const void* v, int32_t q_budget, int32_t kv_budget,
                                  float softmax_scale, void* out, int32_t* sel_idx_opt,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* quoka_strerror(quoka_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* quoka_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QUOKA_H */
