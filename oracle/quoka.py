"""Plain fp64 CPU oracle of QUOKA's per-chunk hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and imports nothing from it.

Every value is computed in float64 from the plain definitions, one
(sequence, KV head) at a time, with NumPy matmuls as the only library steps.
Inputs given in bf16 or fp32 are up-cast exactly, so the oracle sees the very
values the GPU reads.

Sources (the pages this follows):
  [SUM]  "QUOKA: Query-Oriented KV Selection For Efficient LLM Prefill",
         paper summary at hw-hk.tistory.com/367. Sections used: Background >
         Chunked prefill; QUOKA Method > Query Subselection, Scoring via Cosine
         Similarity, Aggregation Across Queries and KV Groups, Chunked Prefill
         with QUOKA.
  [EXP]  "QUOKA Explained: Choosing Which KV History Attention Should Read"
         (reactapp.top). Sections used: "Pick the queries that disagree with
         the crowd", "Letting those queries score the history", "Why take the
         maximum", "From scores to a smaller KV set", "A wrinkle: grouped-query
         attention", "MEAN and MAX do different jobs".

Readings taken where the pages are silent or garbled (the display equations
and both algorithm boxes were lost from the pages):
  * selection is per (sequence, KV head); the KV head's G query heads share it;
  * the vector that stands for token t in subselection is g_t, the mean of the
    token's unit-length query heads of the group (with G = 1: the unit query);
  * MAX over selected tokens is taken of the MEAN over the group's heads;
  * g is not re-normalised before scoring, so g . unit(k) equals the mean of
    the per-head cosines exactly;
  * ties go to the lower token / key index, which makes every selection unique;
  * the causal mask includes the diagonal (token t sees itself) and every
    selected history key is visible to every chunk query;
  * softmax scale 1/sqrt(d) unless given;
  * the chunk's own keys are always attended (causally) and never selected
    over; budgets larger than the data clamp to the data; unit(0) = 0.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against the
pages' worked examples, closed forms, brute-force enumeration and library
routines (torch SDPA in float64). End-to-end values beyond those pins are
"parity unpinned": the pages print no numbers for a whole run.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "unit", "cosine_matrix", "group_query", "query_cosines",
    "lowest_cosine_queries", "key_scores", "top_b_keys", "attend_rows",
    "attend_chunk", "select_for_head", "prefill_chunk", "effective_budgets",
    "prefill_prompt", "VARIANTS", "global_query_cosines", "select_for_sequence",
]

# QUOKA and the baselines the pages set it against (see select_for_sequence).
VARIANTS = ("quoka", "dot", "mean_queries", "mean_query", "per_head", "global")


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def unit(x) -> np.ndarray:
    """Rows (last axis) scaled to unit length; an all-zero row stays zero.

    [SUM] Scoring via Cosine Similarity: cosine similarity normalises vectors
    to unit length. Zero vectors have no direction; we map them to zero, so any
    cosine that involves one is 0.
    """
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    safe = np.where(n > 0.0, n, 1.0)
    return np.where(n > 0.0, x / safe, 0.0)


def cosine_matrix(a, b) -> np.ndarray:
    """cos(a_i, b_j) for rows a [n, d] and b [m, d] -> [n, m].

    [SUM] Scoring via Cosine Similarity: cosine replaces the raw dot product,
    is scale free and bounded in [-1, 1].
    """
    return unit(a) @ unit(b).T


def group_query(q_heads) -> np.ndarray:
    """Pre-aggregated query: the mean of the unit-length query heads.

    q_heads: [..., G, d] (the G query heads that share one KV head)
    returns: [..., d]

    [SUM] Aggregation Across Queries and KV Groups (pre-aggregation): with
    queries normalised first, averaging them across the KV group gives the
    group-mean score in one product. [EXP] "A wrinkle: grouped-query attention":
    average the normalised query heads first, then score once.
    """
    return np.mean(unit(q_heads), axis=-2)


def query_cosines(q_grp):
    """Steps 1-4 of subselection for one (sequence, KV head).

    q_grp: [C, G, d] chunk queries of the group's heads.
    returns (g [C, d], M [d], c [C]) with g_t the token's group query,
    M = mean_t g_t the chunk's mean query and c_t = cos(M, g_t).

    [SUM] Query Subselection: each query is ranked by its (negative) cosine to
    the mean query M_q. [EXP] "Pick the queries that disagree with the crowd":
    compute the chunk's mean query, then each query's cosine to it.
    """
    g = group_query(q_grp)
    if g.shape[0] == 0:  # an empty chunk: no tokens, no mean query
        return g, np.zeros(g.shape[1:]), np.zeros((0,))
    m = np.mean(g, axis=0)
    c = (unit(g) @ unit(m[None, :]).T)[:, 0]
    return g, m, c


def lowest_cosine_queries(c, n_q: int) -> np.ndarray:
    """The n_q tokens least similar to the mean query, ascending token order.

    Order is (c ascending, token ascending); the first min(n_q, C) are kept.
    [SUM] Query Subselection: rank by -CosSim(M_q, q) and keep the top N_q.
    [EXP] "Pick the queries that disagree with the crowd": keep the lowest.
    """
    c = _f64(c)
    n = min(int(n_q), c.shape[0])
    t = np.arange(c.shape[0])
    order = np.lexsort((t, c))  # primary key c, then t
    return np.sort(order[:n])


def key_scores(q_sel, k, *, sim: str = "cos", query_agg: str = "max",
               head_agg: str = "mean") -> np.ndarray:
    """Aggregated score of every history key for one (sequence, KV head).

    q_sel: [n, G, d] the selected tokens' query heads (original, un-averaged)
    k:     [L, d] the KV head's history keys
    returns s [L].

    Computed in the direct form: per-head similarity, then the mean over the
    G heads, then the max over the n selected tokens:
        s_i = max_t (1/G) sum_j cos(q_{t,j}, k_i)
    [SUM] Scoring via Cosine Similarity; Aggregation Across Queries and KV
    Groups (query axis: maximum; GQA axis: average). [EXP] "Why take the
    maximum", "MEAN and MAX do different jobs".

    The other values of ``sim`` / ``query_agg`` are the baselines the pages
    argue against ([SUM] dot-product scoring; [EXP] averaging over queries).
    """
    q_sel = _f64(q_sel)
    k = _f64(k)
    n, G, _ = q_sel.shape
    L = k.shape[0]
    if n == 0 or L == 0:
        return np.zeros((L,), np.float64)
    per_head = []
    for j in range(G):
        if sim == "cos":
            per_head.append(cosine_matrix(q_sel[:, j, :], k))
        elif sim == "dot":
            per_head.append(q_sel[:, j, :] @ k.T)
        else:
            raise ValueError(sim)
    per_head = np.stack(per_head, axis=0)            # [G, n, L]
    if head_agg == "mean":
        grp = np.mean(per_head, axis=0)              # [n, L]
    elif head_agg == "max":
        grp = np.max(per_head, axis=0)
    else:
        raise ValueError(head_agg)
    if query_agg == "max":
        return np.max(grp, axis=0)
    if query_agg == "mean":
        return np.mean(grp, axis=0)
    raise ValueError(query_agg)


def top_b_keys(s, budget: int) -> np.ndarray:
    """Indices of the min(budget, L) highest scores, returned ascending.

    Order is (s descending, index ascending).
    [EXP] "From scores to a smaller KV set": rank the keys and keep the top
    ones within the sparse-attention budget. [SUM] Attention Sparsity: the
    active cache is the subset the scoring function ranks highest.
    """
    s = _f64(s)
    n = min(int(budget), s.shape[0])
    i = np.arange(s.shape[0])
    order = np.lexsort((i, -s))  # primary key -s, then i
    return np.sort(order[:n])


def attend_rows(q_rows, t_rows, k_sel, v_sel, k_chunk, v_chunk,
                scale: float) -> np.ndarray:
    """Softmax attention of chosen query rows over [selected history | own chunk].

    q_rows [m, d]: query vectors (original heads); t_rows [m]: each row's token
    position inside the chunk. Row r sees every selected key and the chunk's
    keys 0..t_rows[r] (diagonal included). Selecting key i brings value i.

    [SUM] Background > Chunked prefill: chunk i attends to the concatenation
    of the earlier chunks' K/V and its own, with a causal mask inside the
    chunk. [EXP] "From scores to a smaller KV set": values follow the keys.
    [EXP] "MEAN and MAX do different jobs": the original query heads do the
    attention.
    """
    q_rows = _f64(q_rows)
    k_sel, v_sel = _f64(k_sel), _f64(v_sel)
    k_chunk, v_chunk = _f64(k_chunk), _f64(v_chunk)
    out = np.zeros_like(q_rows)
    for r in range(q_rows.shape[0]):
        t = int(t_rows[r])
        keys = np.concatenate([k_sel, k_chunk[: t + 1]], axis=0)
        vals = np.concatenate([v_sel, v_chunk[: t + 1]], axis=0)
        logits = (keys @ q_rows[r]) * scale
        w = np.exp(logits - np.max(logits))
        out[r] = (w @ vals) / np.sum(w)
    return out


def attend_chunk(q_head, k_sel, v_sel, k_chunk, v_chunk, scale):
    """All C rows of one query head at once; same definition as attend_rows.

    q_head [C, d]; k_sel, v_sel [B_eff, d]; k_chunk, v_chunk [C, d] -> [C, d].
    """
    q_head, k_sel, v_sel = _f64(q_head), _f64(k_sel), _f64(v_sel)
    k_chunk, v_chunk = _f64(k_chunk), _f64(v_chunk)
    C = q_head.shape[0]
    Bs = k_sel.shape[0]
    keys = np.concatenate([k_sel, k_chunk], axis=0)
    vals = np.concatenate([v_sel, v_chunk], axis=0)
    logits = (q_head @ keys.T) * scale                       # [C, Bs + C]
    own = np.arange(C)
    visible = np.ones((C, Bs + C), dtype=bool)
    visible[:, Bs:] = own[None, :] <= own[:, None]
    logits = np.where(visible, logits, -np.inf)
    w = np.exp(logits - np.max(logits, axis=1, keepdims=True))
    return (w @ vals) / np.sum(w, axis=1, keepdims=True)


def effective_budgets(C_s: int, L_s: int, n_q: int, budget: int):
    """Per-sequence budgets clamped to the data: (min(n_q, C_s), min(B, L_s))."""
    return min(int(n_q), int(C_s)), min(int(budget), int(L_s))


def select_for_head(q_grp, k, n_q: int, budget: int, **score_kw):
    """QUOKA selection for one (sequence, KV head).

    q_grp: [C, G, d] chunk queries of the group; k: [L, d] history keys.
    returns dict(c=[C], S=[n_q_eff] token ids, s=[L], I=[B_eff] key ids).
    [SUM] QUOKA Method: query subselection, cosine scoring, aggregation, then
    the active KV set is chosen (the procedure of its first algorithm box).
    """
    q_grp = _f64(q_grp)
    _, _, c = query_cosines(q_grp)
    S = lowest_cosine_queries(c, n_q)
    s = key_scores(q_grp[S], k, **score_kw)
    I = top_b_keys(s, budget)
    return {"c": c, "S": S, "s": s, "I": I}


def global_query_cosines(q_seq, num_kv_heads: int) -> np.ndarray:
    """One cosine per token for the whole sequence: the mean over the KV heads
    (in head order) of the per-head cosines c_{t,h} to each head's mean query.

    q_seq: [C, H_q, d] -> [C]. Used by the cross-head ("global") baseline,
    where one token subset serves every KV head. [EXP] "A wrinkle:
    grouped-query attention" speaks of one selected token carrying several
    query-head representations, one group per KV head; the average follows
    the GQA-axis rule of [SUM] "Aggregation Across Queries and KV Groups".
    """
    q_seq = _f64(q_seq)
    C, H_q = q_seq.shape[0], q_seq.shape[1]
    H_kv = int(num_kv_heads)
    G = H_q // H_kv
    acc = np.zeros((C,), np.float64)
    for h in range(H_kv):
        acc = acc + query_cosines(q_seq[:, h * G:(h + 1) * G, :])[2]
    return acc / H_kv


def select_for_sequence(q_seq, k_seq, n_q: int, budget: int, variant: str = "quoka"):
    """Selection for every KV head of one sequence, by QUOKA or a baseline.

    q_seq [C, H_q, d]; k_seq [L, H_kv, d]. Returns one dict per KV head with
    c [C] (that head's cosines), S (kept token ids, ascending), s [L], I.

      quoka        the method (select_for_head).
      per_head     the same scores, which the direct form here already takes
                   head by head; [EXP] "A wrinkle: grouped-query attention"
                   names it as the costly way (each head scored, then averaged).
      dot          scores by raw dot products, max over kept tokens of the mean
                   over the group's heads ([SUM] "Scoring via Cosine
                   Similarity": the scale-dependent QK^T of earlier methods).
      mean_queries mean over kept tokens instead of max ([SUM] "Aggregation
                   Across Queries and KV Groups", query axis; [EXP] "Why take
                   the maximum").
      mean_query   no subselection: every chunk token, averaged, scores the keys
                   ([SUM] "Background > Attention Sparsity": single-query
                   methods stretched to many queries by averaging them; [EXP]
                   "One query can choose for itself, but a chunk has
                   thousands"). S is empty.
      global       one kept-token subset per sequence from global_query_cosines,
                   shared by all KV heads; scoring and top-B stay per head.
    """
    if variant not in VARIANTS:
        raise ValueError(variant)
    q_seq, k_seq = _f64(q_seq), _f64(k_seq)
    C, H_q = q_seq.shape[0], q_seq.shape[1]
    H_kv = k_seq.shape[1]
    G = H_q // H_kv
    S_glob = None
    if variant == "global":
        S_glob = lowest_cosine_queries(global_query_cosines(q_seq, H_kv), n_q)
    res = []
    for h in range(H_kv):
        q_grp = q_seq[:, h * G:(h + 1) * G, :]
        k_h = k_seq[:, h, :]
        if variant in ("quoka", "per_head"):
            res.append(select_for_head(q_grp, k_h, n_q, budget))
            continue
        _, _, c = query_cosines(q_grp)
        if variant == "mean_query":
            S = np.zeros((0,), np.int64)
            s = key_scores(q_grp, k_h, query_agg="mean")
        else:
            S = S_glob if variant == "global" else lowest_cosine_queries(c, n_q)
            kw = {"dot": {"sim": "dot"}, "mean_queries": {"query_agg": "mean"},
                  "global": {}}[variant]
            s = key_scores(q_grp[S], k_h, **kw)
        res.append({"c": c, "S": S, "s": s, "I": top_b_keys(s, budget)})
    return res


def prefill_chunk(q, k_hist, v_hist, k_chunk, v_chunk, cu_chunk, cu_hist,
                  num_kv_heads: int, n_q: int, budget: int,
                  scale: float | None = None, *, heads=None,
                  attention: bool = True, variant: str | None = None, **score_kw):
    """The whole per-chunk hot path over a batch of ragged sequences.

    Layouts (token-major, as the library takes them):
      q [sum C, H_q, d]; k_hist, v_hist [sum L, H_kv, d];
      k_chunk, v_chunk [sum C, H_kv, d]; cu_chunk, cu_hist [S + 1] offsets.
    Query head j belongs to KV head j // G ([EXP] "A wrinkle: grouped-query
    attention": contiguous groups).

    ``heads`` restricts the work to a list of KV heads (other outputs stay at
    their fill values); ``attention=False`` skips the attention step;
    ``variant`` picks a baseline selection (select_for_sequence) in place of
    QUOKA's.

    returns dict with
      out     [sum C, H_q, d]  float64 (NaN where not computed)
      q_idx   [S, H_kv, n_q]   int64, ascending, -1 padding
      sel_idx [S, H_kv, B]     int64, ascending, -1 padding
      qcos    [H_kv, sum C]    c_t per token
      scores  [H_kv, sum L]    s_i per history key
    """
    q = _f64(q)
    k_hist, v_hist = _f64(k_hist), _f64(v_hist)
    k_chunk, v_chunk = _f64(k_chunk), _f64(v_chunk)
    cu_chunk = np.asarray(cu_chunk, np.int64)
    cu_hist = np.asarray(cu_hist, np.int64)
    n_seq = cu_chunk.shape[0] - 1
    H_q, d = q.shape[1], q.shape[2]
    H_kv = int(num_kv_heads)
    G = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    heads = range(H_kv) if heads is None else list(heads)

    out = np.full(q.shape, np.nan)
    q_idx = np.full((n_seq, H_kv, n_q), -1, np.int64)
    sel_idx = np.full((n_seq, H_kv, budget), -1, np.int64)
    qcos = np.full((H_kv, q.shape[0]), np.nan)
    scores = np.full((H_kv, k_hist.shape[0]), np.nan)

    for sq in range(n_seq):
        c0, c1 = cu_chunk[sq], cu_chunk[sq + 1]
        h0, h1 = cu_hist[sq], cu_hist[sq + 1]
        per_seq = None
        if variant is not None:
            per_seq = select_for_sequence(q[c0:c1], k_hist[h0:h1], n_q, budget, variant)
        for h in heads:
            q_grp = q[c0:c1, h * G:(h + 1) * G, :]
            k_h = k_hist[h0:h1, h, :]
            if per_seq is not None:
                r = per_seq[h]
            else:
                r = select_for_head(q_grp, k_h, n_q, budget, **score_kw)
            qcos[h, c0:c1] = r["c"]
            scores[h, h0:h1] = r["s"]
            q_idx[sq, h, :r["S"].shape[0]] = r["S"]
            sel_idx[sq, h, :r["I"].shape[0]] = r["I"]
            if not attention or c1 == c0:
                continue
            ks, vs = k_h[r["I"]], v_hist[h0:h1, h, :][r["I"]]
            for j in range(h * G, (h + 1) * G):
                out[c0:c1, j, :] = attend_chunk(
                    q[c0:c1, j, :], ks, vs, k_chunk[c0:c1, h, :],
                    v_chunk[c0:c1, h, :], scale)
    return {"out": out, "q_idx": q_idx, "sel_idx": sel_idx,
            "qcos": qcos, "scores": scores}


def prefill_prompt(q, k, v, chunk_len: int, num_kv_heads: int, n_q: int, budget: int,
                   scale: float | None = None, **score_kw):
    """A whole prompt of one sequence through chunked prefill with QUOKA.

    [SUM] "Background > Chunked prefill": the prompt of T tokens is split into
    ceil(T / B_cp) consecutive chunks of B_cp tokens (the last may be
    shorter); chunk i attends to the keys and values of every earlier chunk
    concatenated with its own, under a causal mask inside the chunk.
    [SUM] "QUOKA Method" (the chunked-prefill algorithm at its end) and [EXP]
    "Chunked prefill": for each new chunk QUOKA selects the active history
    KVs from all earlier tokens (chunk 0 has no history) and passes them with
    the chunk's own KVs to the attention; nothing is evicted, the next chunk
    selects again from the whole history.

    q [T, H_q, d]; k, v [T, H_kv, d] (the keys and values the prompt writes,
    chunk by chunk, into the cache). Returns dict with
      out     [T, H_q, d] float64
      sel_idx [n_chunks, H_kv, budget] int64 (per chunk, indices into k[:start])
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T = q.shape[0]
    n_chunks = -(-T // chunk_len)
    out = np.empty(q.shape)
    sel = np.full((n_chunks, int(num_kv_heads), budget), -1, np.int64)
    for i in range(n_chunks):
        a, b = i * chunk_len, min(T, (i + 1) * chunk_len)
        r = prefill_chunk(q[a:b], k[:a], v[:a], k[a:b], v[a:b], [0, b - a], [0, a],
                          num_kv_heads, n_q, budget, scale, **score_kw)
        out[a:b] = r["out"]
        sel[i] = r["sel_idx"][0]
    return {"out": out, "sel_idx": sel}
