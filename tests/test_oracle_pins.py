"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: the
numbers printed in the pages' worked examples (tests/golden), closed forms,
brute-force enumeration and a library routine (torch SDPA in float64).
The last test plants mistakes in the oracle and asserts a pin catches each.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import quoka as oq

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "worked_examples.json")))


# ---------------------------------------------------------------- helpers
def _table_vectors(table):
    """Unit queries with prescribed cosines to orthonormal keys e_0..e_{m-1}.

    Row r of the table becomes q_r = sum_i T[r,i] e_i + sqrt(1 - |T_r|^2) e_{m+r},
    so cos(q_r, e_i) = T[r, i] exactly (up to rounding).
    """
    T = np.asarray(table, np.float64)
    n, m = T.shape
    d = m + n
    q = np.zeros((n, d))
    q[:, :m] = T
    for r in range(n):
        q[r, m + r] = math.sqrt(1.0 - np.sum(T[r] ** 2))
    k = np.eye(d)[:m]
    return q, k


def _sdpa(q, k, v, mask, scale):
    """torch's attention in float64 on CPU: q [m,d], k/v [n,d], mask [m,n] bool."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(mask)[None, None],
        scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- pins
def pin_subselection_worked_example():
    ex = GOLD["subselection"]
    got = oracle.lowest_cosine_queries(np.array(ex["cos_to_mean"]), ex["keep"])
    assert got.tolist() == ex["kept"], got


def pin_query_cosine_closed_form():
    # tokens e1, e1, e2 (G = 1): M = (2 e1 + e2)/3, |M| = sqrt(5)/3,
    # cos(M, e1) = 2/sqrt(5), cos(M, e2) = 1/sqrt(5); the e2 token is kept.
    q = np.zeros((3, 1, 4))
    q[0, 0, 0] = 2.0
    q[1, 0, 0] = 0.5          # norms differ: normalisation must remove them
    q[2, 0, 1] = 7.0
    g, m, c = oracle.query_cosines(q)
    np.testing.assert_allclose(c, [2 / math.sqrt(5), 2 / math.sqrt(5),
                                   1 / math.sqrt(5)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(m, [2 / 3, 1 / 3, 0, 0], atol=1e-15)
    assert oracle.lowest_cosine_queries(c, 1).tolist() == [2]


def pin_group_query_closed_form():
    # heads (3,4) and (0,2): unit -> (.6,.8), (0,1); mean -> (.3,.9)
    q = np.array([[[3.0, 4.0], [0.0, 2.0]]])
    np.testing.assert_allclose(oracle.group_query(q), [[0.3, 0.9]], atol=1e-15)


def pin_score_table_max():
    ex = GOLD["score_table"]
    q, k = _table_vectors(ex["cos"])
    k = k * np.array([[3.0], [0.25], [9.0], [1.5]])   # key scale must not matter
    s = oracle.key_scores(q[:, None, :], k)
    np.testing.assert_allclose(s, ex["max_over_queries"], atol=1e-14)
    s_mean = oracle.key_scores(q[:, None, :], k, query_agg="mean")
    np.testing.assert_allclose(s_mean[0], ex["mean_over_queries_K1"], atol=1e-14)


def pin_k50_max():
    ex = GOLD["k50"]
    q, k = _table_vectors(np.array(ex["cos"])[:, None])
    np.testing.assert_allclose(oracle.key_scores(q[:, None, :], k), [ex["max"]],
                               atol=1e-14)


def pin_gqa_mean_over_heads():
    # one token, heads e1 and e2, key e1: per-head cosines 1 and 0 -> mean .5
    q = np.zeros((1, 2, 3))
    q[0, 0, 0] = 5.0
    q[0, 1, 1] = 0.1
    k = np.array([[2.0, 0.0, 0.0], [0.0, 0.0, 1.0]])
    np.testing.assert_allclose(oracle.key_scores(q, k), [0.5, 0.0], atol=1e-15)


def pin_pre_aggregation_identity():
    # mean of per-head cosines == (mean of unit heads) . unit(k)
    rng = np.random.default_rng(1)
    q = rng.standard_normal((6, 4, 16)) * rng.uniform(0.1, 5, (6, 4, 1))
    k = rng.standard_normal((40, 16)) * rng.uniform(0.1, 5, (40, 1))
    g = np.mean(q / np.linalg.norm(q, axis=-1, keepdims=True), axis=1)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    np.testing.assert_allclose(oracle.key_scores(q, k), np.max(g @ kn.T, axis=0),
                               atol=1e-13)


def pin_top_keys_worked_example():
    ex = GOLD["top_keys"]
    s = np.full(ex["num_keys"], ex["score_tail"])
    s[:len(ex["scores_head"])] = ex["scores_head"]
    assert oracle.top_b_keys(s, ex["budget"]).tolist() == ex["selected"]


def _brute_force_top(s, b):
    """The unique size-b subset whose every member ranks above every non-member
    under (score desc, index asc)."""
    n = len(s)
    rank_key = lambda i: (-s[i], i)
    found = []
    for sub in itertools.combinations(range(n), b):
        rest = [i for i in range(n) if i not in sub]
        if not rest or not sub or \
                max(rank_key(i) for i in sub) < min(rank_key(i) for i in rest):
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


def pin_top_keys_brute_force():
    rng = np.random.default_rng(2)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        s = rng.choice([-0.5, 0.1, 0.2, 0.3], size=n)   # many ties
        for b in range(0, n + 1):
            assert oracle.top_b_keys(s, b).tolist() == _brute_force_top(s, b)


def pin_lowest_queries_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(60):
        n = int(rng.integers(1, 11))
        c = rng.choice([-0.3, 0.0, 0.4, 0.9], size=n)
        for b in range(0, n + 1):
            want = _brute_force_top(-c, b)
            assert oracle.lowest_cosine_queries(c, b).tolist() == want


def pin_attention_dense_when_budget_covers_history():
    """B >= L: the path is exactly dense causal attention over [K_<i | K_i]."""
    rng = np.random.default_rng(4)
    C, L, H_q, H_kv, d = 7, 9, 4, 2, 8
    q = rng.standard_normal((C, H_q, d))
    kh, vh = rng.standard_normal((L, H_kv, d)), rng.standard_normal((L, H_kv, d))
    kc, vc = rng.standard_normal((C, H_kv, d)), rng.standard_normal((C, H_kv, d))
    r = oracle.prefill_chunk(q, kh, vh, kc, vc, [0, C], [0, L], H_kv, n_q=3,
                             budget=L + 5)
    mask = np.ones((C, L + C), bool)
    mask[:, L:] = np.tril(np.ones((C, C), bool))
    for j in range(H_q):
        h = j // (H_q // H_kv)
        want = _sdpa(q[:, j], np.concatenate([kh[:, h], kc[:, h]]),
                     np.concatenate([vh[:, h], vc[:, h]]), mask, 1 / math.sqrt(d))
        np.testing.assert_allclose(r["out"][:, j], want, atol=1e-12)
    assert r["sel_idx"][0, 0].tolist() == list(range(L)) + [-1] * 5


def pin_attention_no_history_is_causal_self_attention():
    rng = np.random.default_rng(5)
    C, d = 6, 8
    q = rng.standard_normal((C, 1, d))
    kc, vc = rng.standard_normal((C, 1, d)), rng.standard_normal((C, 1, d))
    e = np.zeros((0, 1, d))
    r = oracle.prefill_chunk(q, e, e, kc, vc, [0, C], [0, 0], 1, 4, 4, scale=0.3)
    tt = lambda a: torch.from_numpy(a)[None, None]
    want = torch.nn.functional.scaled_dot_product_attention(
        tt(q[:, 0]), tt(kc[:, 0]), tt(vc[:, 0]), is_causal=True, scale=0.3)
    np.testing.assert_allclose(r["out"][:, 0], want[0, 0].numpy(), atol=1e-12)


def pin_attention_special_cases():
    rng = np.random.default_rng(6)
    d = 5
    kc, vc = rng.standard_normal((4, d)), rng.standard_normal((4, d))
    ks, vs = rng.standard_normal((3, d)), rng.standard_normal((3, d))
    # one visible key: token 0 with no history sees only its own value
    o = oracle.attend_rows(rng.standard_normal((1, d)), [0], ks[:0], vs[:0], kc, vc, 1.0)
    np.testing.assert_allclose(o[0], vc[0], atol=1e-15)
    # equal logits (zero query): the mean of the visible values
    o = oracle.attend_rows(np.zeros((1, d)), [2], ks, vs, kc, vc, 1.0)
    np.testing.assert_allclose(o[0], np.concatenate([vs, vc[:3]]).mean(0), atol=1e-15)
    # values follow keys, order of the selected set does not matter
    ex = GOLD["values_follow_keys"]
    qr = rng.standard_normal((2, d))
    a = oracle.attend_rows(qr, [1, 3], ks, vs, kc, vc, 0.7)
    p = ex["keys_kept"]
    b = oracle.attend_rows(qr, [1, 3], ks[p], vs[ex["values_kept"]], kc, vc, 0.7)
    np.testing.assert_allclose(a, b, atol=1e-14)


def pin_scale_invariance():
    """Positive rescaling of any query head or key leaves the selection unchanged."""
    rng = np.random.default_rng(7)
    C, L, H_q, H_kv, d = 12, 30, 4, 2, 8
    q = rng.standard_normal((C, H_q, d))
    kh = rng.standard_normal((L, H_kv, d))
    kc, vc, vh = (rng.standard_normal((n, H_kv, d)) for n in (C, C, L))
    r1 = oracle.prefill_chunk(q, kh, vh, kc, vc, [0, C], [0, L], H_kv, 3, 7,
                              attention=False)
    q2 = q * rng.uniform(0.05, 20.0, (C, H_q, 1))
    k2 = kh * rng.uniform(0.05, 20.0, (L, H_kv, 1))
    r2 = oracle.prefill_chunk(q2, k2, vh, kc, vc, [0, C], [0, L], H_kv, 3, 7,
                              attention=False)
    np.testing.assert_allclose(r1["qcos"], r2["qcos"], atol=1e-12)
    np.testing.assert_allclose(r1["scores"], r2["scores"], atol=1e-12)
    assert (r1["sel_idx"] == r2["sel_idx"]).all()
    assert (r1["q_idx"] == r2["q_idx"]).all()


def pin_needle_recovered():
    """A key aligned with an outlier query (forced into the kept set) is selected."""
    rng = np.random.default_rng(8)
    C, L, d = 32, 200, 16
    common = rng.standard_normal(d)
    q = common[None, :] + 0.05 * rng.standard_normal((C, d))
    out_tok = 11
    q[out_tok] = rng.standard_normal(d)
    q[out_tok] -= q[out_tok] @ common / (common @ common) * common  # orthogonal
    k = rng.standard_normal((L, d))
    needle = 57
    k[needle] = 3 * math.sqrt(d) * q[out_tok] / np.linalg.norm(q[out_tok]) \
        + rng.standard_normal(d)
    r = oracle.select_for_head(q[:, None, :], k, n_q=1, budget=1)
    assert r["S"].tolist() == [out_tok]
    assert r["I"].tolist() == [needle]


def pin_clamped_budgets():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((5, 2, 4))
    k = rng.standard_normal((6, 4))
    r = oracle.select_for_head(q, k, n_q=99, budget=99)
    assert r["S"].tolist() == list(range(5))
    assert r["I"].tolist() == list(range(6))
    r = oracle.select_for_head(q, k[:0], n_q=2, budget=3)
    assert r["I"].tolist() == [] and r["s"].shape == (0,)


def pin_zero_vectors():
    q = np.zeros((4, 1, 3))
    g, m, c = oracle.query_cosines(q)
    assert np.all(c == 0) and np.all(m == 0)
    assert oracle.lowest_cosine_queries(c, 2).tolist() == [0, 1]
    k = np.array([[0.0, 0.0, 0.0], [1.0, 0.0, 0.0]])
    qq = np.array([[[-1.0, 0.0, 0.0]]])
    np.testing.assert_allclose(oracle.key_scores(qq, k), [0.0, -1.0])


def pin_chunking_example():
    """The chunk partition used by the chunked-prefill loop (3000 tokens, 1000 per chunk)."""
    ex = GOLD["chunking"]
    T, Bcp = ex["prompt_tokens"], ex["chunk"]
    nb = math.ceil(T / Bcp)
    chunks = [[i * Bcp, min((i + 1) * Bcp, T) - 1] for i in range(nb)]
    assert chunks == ex["chunks"]
    assert [c[0] for c in chunks] == ex["history_before_chunk"]


def _dense_causal(q, k, v):
    """Dense causal attention over a whole prompt by torch's scaled dot-product attention
    (an independent library routine), GQA by repeating each KV head over its query heads."""
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.permute(1, 0, 2).numpy()


def pin_prompt_with_full_budget_is_dense_causal_attention():
    """Keeping every history key, chunked prefill reproduces dense causal attention over the
    whole prompt (the chunk masks and the history concatenation together are the causal mask)."""
    rng = np.random.default_rng(11)
    T, Hq, Hkv, d = 257, 4, 2, 16
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    for chunk in (64, 100, 257):
        r = oracle.prefill_prompt(q, k, v, chunk, Hkv, 8, T)
        np.testing.assert_allclose(r["out"], _dense_causal(q, k, v), atol=1e-12)
        n = -(-T // chunk)
        assert r["sel_idx"].shape == (n, Hkv, T)
        for i in range(n):  # chunk i keeps exactly its i*chunk history keys, ascending
            kept = r["sel_idx"][i, 0]
            assert kept[: i * chunk].tolist() == list(range(i * chunk))
            assert np.all(kept[i * chunk:] == -1)


def pin_prompt_chunk_zero_and_single_chunk_ignore_the_budget():
    """Chunk 0 has no history, so a prompt that fits one chunk is dense causal attention
    whatever the budgets; with several chunks and a small budget, chunk 0 still is."""
    rng = np.random.default_rng(12)
    T, Hq, Hkv, d = 80, 2, 1, 8
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    dense = _dense_causal(q, k, v)
    np.testing.assert_allclose(oracle.prefill_prompt(q, k, v, T, Hkv, 1, 1)["out"], dense,
                               atol=1e-12)
    r = oracle.prefill_prompt(q, k, v, 32, Hkv, 2, 3)
    np.testing.assert_allclose(r["out"][:32], dense[:32], atol=1e-12)
    assert not np.allclose(r["out"][64:], dense[64:])  # later chunks see only 3 history keys


# ------------------------------------------------ baselines (select_for_sequence)
def pin_variant_dot_closed_form():
    """Raw dot products: max over tokens of the mean over the group's heads."""
    q = np.array([[[3.0, 4.0], [0.0, 2.0]],      # token 0, heads 0 and 1
                  [[0.0, -1.0], [1.0, 0.0]]])    # token 1
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[2.0, 0.0]]])   # [L=3, H_kv=1, d]
    r = oracle.select_for_sequence(q, k, 2, 2, "dot")[0]
    # key 0: means 1.5, 0.5; key 1: 3, -0.5; key 2 (key 0 doubled): 3, 1
    np.testing.assert_allclose(r["s"], [1.5, 3.0, 3.0], atol=1e-15)
    assert r["I"].tolist() == [1, 2]
    r_cos = oracle.select_for_sequence(q, k, 2, 2, "quoka")[0]
    assert r_cos["s"][0] == pytest.approx(r_cos["s"][2], abs=1e-15)  # cosine ignores scale


def pin_variant_mean_queries_worked_example():
    """The score table of the worked example averaged over its three queries."""
    ex = GOLD["score_table"]
    q, k = _table_vectors(ex["cos"])
    r = oracle.select_for_sequence(q[:, None, :], k[:, None, :], 3, 2, "mean_queries")[0]
    np.testing.assert_allclose(r["s"][0], ex["mean_over_queries_K1"], atol=1e-14)
    # the other columns of the printed table, averaged by hand
    np.testing.assert_allclose(r["s"], [0.40, 0.35, 1.30 / 3, 0.15], atol=1e-14)
    assert r["S"].tolist() == [0, 1, 2] and r["I"].tolist() == [0, 2]


def pin_variant_mean_query_closed_form():
    """One query, the chunk's mean: tokens e1, e1, e2 (norms 2, 0.5, 7) give
    per-key mean cosines 2/3 (e1), 1/3 (e2) and 1/sqrt(2) ((e1 + e2) scaled)."""
    q = np.zeros((3, 1, 4))
    q[0, 0, 0], q[1, 0, 0], q[2, 0, 1] = 2.0, 0.5, 7.0
    k = np.zeros((3, 1, 4))
    k[0, 0, 0], k[1, 0, 1] = 3.0, 1.0
    k[2, 0, :2] = 5.0
    r = oracle.select_for_sequence(q, k, 1, 1, "mean_query")[0]
    np.testing.assert_allclose(r["s"], [2 / 3, 1 / 3, 1 / math.sqrt(2)], atol=1e-15)
    assert r["S"].shape == (0,) and r["I"].tolist() == [2]
    # QUOKA with the one kept token (e2, the least like the mean) scores e2 highest
    rq = oracle.select_for_sequence(q, k, 1, 1, "quoka")[0]
    assert rq["S"].tolist() == [2] and rq["I"].tolist() == [1]


def _two_head_tokens():
    # head 0: tokens e1 (x2), e1 (x0.5), e2 (x7); head 1: e2, e1, e1 (G = 1)
    q = np.zeros((3, 2, 4))
    q[0, 0, 0], q[1, 0, 0], q[2, 0, 1] = 2.0, 0.5, 7.0
    q[0, 1, 1], q[1, 1, 0], q[2, 1, 0] = 1.0, 3.0, 1.0
    k = np.zeros((2, 2, 4))
    k[0, :, 0] = 1.0
    k[1, :, 1] = 1.0
    return q, k


def pin_variant_global_closed_form():
    """Per-head cosines (2, 2, 1)/sqrt(5) and (1, 2, 2)/sqrt(5) average to
    (1.5, 2, 1.5)/sqrt(5); the shared lowest token is 0 (tie to the lower)."""
    q, k = _two_head_tokens()
    r5 = math.sqrt(5.0)
    np.testing.assert_allclose(oracle.global_query_cosines(q, 2),
                               [1.5 / r5, 2 / r5, 1.5 / r5], atol=1e-15)
    glob = oracle.select_for_sequence(q, k, 1, 1, "global")
    per = oracle.select_for_sequence(q, k, 1, 1, "quoka")
    assert [r["S"].tolist() for r in glob] == [[0], [0]]
    assert [r["S"].tolist() for r in per] == [[2], [0]]
    np.testing.assert_allclose(glob[0]["s"], [1.0, 0.0], atol=1e-15)   # token 0 of head 0 is e1
    np.testing.assert_allclose(per[0]["s"], [0.0, 1.0], atol=1e-15)    # token 2 of head 0 is e2
    assert [r["S"].tolist() for r in oracle.select_for_sequence(q, k, 2, 1, "global")] == \
        [[0, 2], [0, 2]]


def pin_variant_global_with_one_kv_head_is_quoka():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((9, 3, 8))
    k = rng.standard_normal((20, 1, 8))
    a = oracle.select_for_sequence(q, k, 4, 6, "global")[0]
    b = oracle.select_for_head(q, k[:, 0], 4, 6)
    assert a["S"].tolist() == b["S"].tolist() and a["I"].tolist() == b["I"].tolist()
    np.testing.assert_allclose(a["s"], b["s"], atol=1e-15)


def pin_effective_budgets_match_the_selections():
    # the clamp the checks use equals the sizes select_for_head actually returns (its
    # sorts slice to min(n_q, C) and min(B, L)), over budgets below, at and above the data
    rng = np.random.default_rng(11)
    for C, L in ((5, 9), (1, 1), (7, 0), (3, 40), (12, 12)):
        q = rng.standard_normal((C, 2, 4))
        k = rng.standard_normal((L, 4))
        for nq, b in ((1, 1), (4, 8), (C, L if L else 1), (C + 3, L + 5), (50, 2)):
            r = oracle.select_for_head(q, k, nq, b)
            assert oracle.effective_budgets(C, L, nq, b) == (r["S"].shape[0], r["I"].shape[0])


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes
def _mutations():
    orig_unit = oq.unit
    orig_lexsort = np.lexsort

    def no_norm(x):
        return np.asarray(x, np.float64)

    def key_scores_mean(q_sel, k, **kw):
        kw["query_agg"] = "mean"
        return orig_key_scores(q_sel, k, **kw)

    def key_scores_dot(q_sel, k, **kw):
        kw["sim"] = "dot"
        return orig_key_scores(q_sel, k, **kw)

    def key_scores_headmax(q_sel, k, **kw):
        kw["head_agg"] = "max"
        return orig_key_scores(q_sel, k, **kw)

    def highest_cos(c, n_q):
        return orig_lowest(-np.asarray(c), n_q)

    def lowest_scores(s, b):
        return orig_top(-np.asarray(s), b)

    def causal_strict(q_rows, t_rows, k_sel, v_sel, k_chunk, v_chunk, scale):
        t = np.asarray(t_rows)
        return orig_attend(q_rows, np.maximum(t - 1, 0), k_sel, v_sel, k_chunk,
                           v_chunk, scale)

    def chunk_strict(q_head, k_sel, v_sel, k_chunk, v_chunk, scale):
        m = q_head.shape[0]
        return causal_strict(q_head, np.arange(m), k_sel, v_sel, k_chunk, v_chunk, scale)

    def tie_high_index(s, b):
        s = np.asarray(s, np.float64)
        i = np.arange(s.shape[0])
        return np.sort(orig_lexsort((-i, -s))[:min(b, s.shape[0])])

    def global_head0(q_seq, num_kv_heads):
        q_seq = np.asarray(q_seq, np.float64)
        G = q_seq.shape[1] // num_kv_heads
        return orig_query_cosines(q_seq[:, :G, :])[2]

    orig_query_cosines = oq.query_cosines
    orig_key_scores, orig_lowest, orig_top = oq.key_scores, oq.lowest_cosine_queries, oq.top_b_keys
    orig_attend = oq.attend_rows
    return {
        "no_normalisation": ("unit", no_norm),
        "mean_over_queries": ("key_scores", key_scores_mean),
        "dot_product_scores": ("key_scores", key_scores_dot),
        "max_over_heads": ("key_scores", key_scores_headmax),
        "keep_highest_cosine": ("lowest_cosine_queries", highest_cos),
        "keep_lowest_scores": ("top_b_keys", lowest_scores),
        "tie_to_higher_index": ("top_b_keys", tie_high_index),
        "mask_without_diagonal": ("attend_rows", causal_strict),
        "chunk_mask_without_diagonal": ("attend_chunk", chunk_strict),
        "global_from_first_head_only": ("global_query_cosines", global_head0),
        "budgets_not_clamped": ("effective_budgets", lambda C, L, nq, b: (int(nq), int(b))),
    }


@pytest.mark.parametrize("name", sorted(_mutations().keys()))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = _mutations()[name]
    monkeypatch.setattr(oq, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
