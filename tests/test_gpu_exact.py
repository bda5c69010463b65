"""GPU selections near their boundaries, where the fp32 values alone cannot
decide: clusters of near-duplicate history keys (or chunk tokens) whose fp64
scores (cosines) differ by about 1e-7 relative, planted so that the B-th key
(the N_q-th token) falls inside the cluster, and exact duplicates (equal
values, decided by the lower index). The library re-evaluates such members in
fp64, so its kept sets must equal the oracle's exactly.

The budgets are placed with the oracle, on the CPU; every expected value is
the oracle's.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_kv_amd as cpk
import oracle
from workloads import make_case

from gpu_check import upload, score_bound, QCOS_TOL

pytestmark = pytest.mark.gpu


def _rank_desc(s):
    return np.lexsort((np.arange(s.shape[0]), -s))


def _plant_key_cluster(w, rng, h, base, m, rel):
    """m copies of history key `base` (head h) at random other positions, each coordinate
    scaled by (1 + rel * N(0, 1)); rel = 0 gives exact duplicates."""
    L = w.k_hist.shape[0]
    pos = rng.choice(np.setdiff1d(np.arange(L), [base]), size=m, replace=False)
    row = w.k_hist[base, h].astype(np.float64)
    for p in pos:
        w.k_hist[p, h] = (row * (1.0 + rel * rng.standard_normal(row.shape))).astype(np.float32)
    return np.concatenate([[base], pos])


@pytest.mark.parametrize("dtype,rel", [("fp32", 3e-6), ("bf16", 0.0)])
def test_key_boundary_cluster_matches_oracle_exactly(dtype, rel):
    w = make_case([(96, 4000)], 4, 2, 64, dtype, 8, 256, seed=77, name=f"key_cluster_{dtype}")
    rng = np.random.default_rng(78)
    G = w.num_q_heads // w.num_kv_heads
    q = w.q.astype(np.float64)
    B = w.budget
    clusters = {}
    for h in range(w.num_kv_heads):
        q_grp = q[:, h * G:(h + 1) * G]
        r = oracle.select_for_head(q_grp, w.k_hist[:, h].astype(np.float64), w.n_q, B)
        base = int(_rank_desc(r["s"])[B - 20])
        clusters[h] = _plant_key_cluster(w, rng, h, base, 39, rel)
    print(f"[gpu] key boundary cluster {dtype}", flush=True)
    shape, t = upload(w)
    sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, B, want_q_idx=True, want_scores=True)
    torch.cuda.synchronize()
    r = {k: v.cpu().numpy() for k, v in sel.items() if v is not None}
    for h in range(w.num_kv_heads):
        S_gpu = r["q_idx"][0, h][: w.n_q].astype(np.int64)
        q_grp = q[:, h * G:(h + 1) * G]
        S_or = oracle.lowest_cosine_queries(oracle.query_cosines(q_grp)[2], w.n_q)
        assert np.array_equal(S_gpu, S_or), f"head {h}: kept queries differ"
        s_or = oracle.key_scores(q_grp[S_or], w.k_hist[:, h].astype(np.float64))
        I_or = oracle.top_b_keys(s_or, B)
        kept = np.isin(clusters[h], I_or).sum()
        assert 0 < kept < clusters[h].shape[0], f"head {h}: the cluster does not straddle"
        order = np.sort(s_or)[::-1]
        if rel > 0:  # distinct values: the boundary gap is above the keys' 2^-28 resolution
            assert order[B - 1] - order[B] > 1e-8 * abs(order[B - 1])
        I_gpu = r["sel_idx"][0, h][:B].astype(np.int64)
        s_gpu = r["scores"][h].astype(np.float64)
        eps = score_bound(dtype, w.head_dim)
        assert np.max(np.abs(s_gpu - s_or)) <= eps
        fp32_rule = oracle.top_b_keys(s_gpu, B)
        print(f"[gpu] head {h}: cluster kept {kept}/{clusters[h].shape[0]}, the fp32 scores "
              f"alone would differ in {len(set(fp32_rule) ^ set(I_or))} keys", flush=True)
        assert np.array_equal(I_gpu, I_or), (
            f"head {h}: kept keys differ from the oracle: {sorted(set(I_gpu) ^ set(I_or))[:8]}")


@pytest.mark.parametrize("dtype,rel", [("fp32", 3e-6), ("bf16", 0.0)])
def test_query_boundary_cluster_matches_oracle_exactly(dtype, rel):
    # one KV head of four query heads; the token least similar to the mean query is copied to
    # 19 other positions (scaled by 1 + rel N(0, 1) per coordinate) and its negation to 19 more,
    # so that the mean query hardly moves and the 20 copies hold the 20 lowest cosines; with
    # N_q = 10 the boundary falls inside them
    w = make_case([(300, 1000)], 4, 1, 64, dtype, 10, 64, seed=79, name=f"query_cluster_{dtype}")
    rng = np.random.default_rng(80)
    C = w.q.shape[0]
    c = oracle.query_cosines(w.q.astype(np.float64))[2]
    base = int(np.argmin(c))
    pos = rng.choice(np.setdiff1d(np.arange(C), [base]), size=38, replace=False)
    row = w.q[base].astype(np.float64)
    for i, p in enumerate(pos):
        sign = 1.0 if i < 19 else -1.0
        w.q[p] = (sign * row * (1.0 + rel * rng.standard_normal(row.shape))).astype(np.float32)
    cluster = np.concatenate([[base], pos[:19]])
    print(f"[gpu] query boundary cluster {dtype}", flush=True)
    shape, t = upload(w)
    sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, w.budget, want_q_idx=True,
                     want_qcos=True)
    torch.cuda.synchronize()
    r = {k: v.cpu().numpy() for k, v in sel.items() if v is not None}
    c_or = oracle.query_cosines(w.q.astype(np.float64))[2]
    S_or = oracle.lowest_cosine_queries(c_or, w.n_q)
    kept = np.isin(cluster, S_or).sum()
    assert 0 < kept < cluster.shape[0], "the cluster does not straddle the boundary"
    order = np.sort(c_or)
    if rel > 0:  # distinct values: the boundary gap is above the tokens' 2^-26 resolution
        assert order[w.n_q] - order[w.n_q - 1] > 4e-8 * abs(order[w.n_q - 1])
    c_gpu = r["qcos"][0].astype(np.float64)
    assert np.max(np.abs(c_gpu - c_or)) <= QCOS_TOL
    S_gpu = r["q_idx"][0, 0][: w.n_q].astype(np.int64)
    fp32_rule = oracle.lowest_cosine_queries(c_gpu, w.n_q)
    print(f"[gpu] cluster kept {kept}/{cluster.shape[0]}, the fp32 cosines alone would differ "
          f"in {len(set(fp32_rule) ^ set(S_or))} tokens", flush=True)
    assert np.array_equal(S_gpu, S_or), (
        f"kept queries differ from the oracle: {sorted(set(S_gpu) ^ set(S_or))}")
