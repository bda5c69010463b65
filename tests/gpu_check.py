"""Helpers for the GPU parity tests: upload a workload, run the library, and
check every stage against the fp64 oracle.

The check is stage-conditioned: each oracle stage after the first runs on the
GPU's own result of the stage before (its kept queries for scoring, its kept
keys for attention), so a legitimate near-tie in one stage cannot cascade
into differences in later ones. Index sets must match the oracle's exactly
except for members whose oracle value lies within 1e-5 relative of the
boundary value (the stated selection tolerance):

* kept queries: |c_t - c_(N_q)| <= 1e-5 |c_(N_q)|;
* kept keys:    |s_i - s_(B)|   <= 1e-5 |s_(B)|.

The library meets this by construction: its fp32 cosines and scores are
within stated bounds (QCOS_TOL, score_bound) of the fp64 values, and every
member within twice that bound of its fp32 boundary value is re-evaluated in
fp64 before the choice. So the GPU's selection must also equal the selection
rule applied to its own fp32 values, except inside that re-evaluation band.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import chunked_prefill_kv_amd as cpk
import oracle

QCOS_TOL = 2.0 ** -22     # |c_gpu - c_oracle|: the library's stated bound on its fp32 cosines
SEL_REL_BAND = 1e-5       # the stated selection tolerance, relative to the boundary value
ATTN_TOL = {"fp32": 1e-4, "bf16": 2e-2}    # max-abs on the attention output


def score_bound(dtype: str, head_dim: int, group: int = 1, per_head: bool = False) -> float:
    """The library's stated bound on |fp32 score - fp64 score| (cosine scores).

    Rows rounded to fp32 (2 u; the per-head baseline's unit rows carry an
    fp32 norm, d/2 + 3 u), the bf16 hi/lo split (2^-18), nt products summed
    in fp32 (2 nt u), and the key norm, its square root and the quotient
    ((d + 4) u), u = 2^-24."""
    u = 2.0 ** -24
    bf = dtype == "bf16"
    gh = group if per_head else 1
    nt = (2 if bf else 1) * head_dim * gh
    rows = (head_dim / 2 + 3 if per_head else 2.0) * u
    row = rows + (2.0 ** -18 * 1.01 if bf else 0.0) + 2 * nt * u * 1.01
    return (row + (head_dim + 4) * u * 1.01) * 1.001


def upload(w, device="cuda"):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = cpk.Shape(w.cu_chunk, w.cu_hist, w.num_q_heads, w.num_kv_heads, w.head_dim,
                      w.dtype, device=device)
    t = {}
    for name in ("q", "k_hist", "v_hist", "k_chunk", "v_chunk"):
        t[name] = torch.from_numpy(getattr(w, name)).to(dt).to(device).contiguous()
    return shape, t


def run_stages(w, shape, t):
    """Stage-wise calls: select (with every optional output), gather, attend."""
    B = w.budget
    sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, B, want_q_idx=True, want_qcos=True,
                     want_scores=True)
    k_sel, v_sel = cpk.gather(shape, t["k_hist"], t["v_hist"], sel["sel_idx"], B)
    out = cpk.chunk_attn(shape, t["q"], k_sel, v_sel, B, t["k_chunk"], t["v_chunk"])
    out_fused = cpk.chunk_attn_gather(shape, t["q"], t["k_hist"], t["v_hist"], sel["sel_idx"], B,
                                      t["k_chunk"], t["v_chunk"])
    torch.cuda.synchronize()
    return {k: (v.cpu().float().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy())
            for k, v in dict(sel, k_sel=k_sel, v_sel=v_sel, out=out, out_fused=out_fused).items()
            if v is not None}


def _band_check(got, want, values, boundary, band, what):
    diff = set(got.tolist()) ^ set(want.tolist())
    bad = [i for i in diff if abs(values[i] - boundary) > band]
    assert not bad, (f"{what}: {len(bad)} members differ outside the tie band "
                     f"(band {band:.3g}, first {bad[:5]}, values "
                     f"{[float(values[i]) for i in bad[:5]]}, boundary {boundary!r})")
    return len(diff)


def _rule_check(got, want, values, boundary, band, what):
    """The GPU's set against the selection rule on its own fp32 values: equal except for
    members within `band` of the GPU's fp32 boundary value (there it decided in fp64)."""
    diff = set(got.tolist()) ^ set(want.tolist())
    bad = [i for i in diff if abs(values[i] - boundary) > band]
    assert not bad, (f"{what}: differs from the selection rule on its own values outside the "
                     f"re-evaluation band ({len(bad)} members, first {bad[:5]})")


def check_selection(w, r, heads=None, seqs=None):
    """Stages 1-4 for the given (sequence, KV head) pairs. Returns tie counts."""
    q = w.q.astype(np.float64)
    kh = w.k_hist.astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    heads = range(w.num_kv_heads) if heads is None else heads
    seqs = range(w.num_seqs) if seqs is None else seqs
    ties = {"q": 0, "k": 0}
    for s in seqs:
        c0, c1 = int(w.cu_chunk[s]), int(w.cu_chunk[s + 1])
        h0, h1 = int(w.cu_hist[s]), int(w.cu_hist[s + 1])
        nq_eff, b_eff = oracle.effective_budgets(c1 - c0, h1 - h0, w.n_q, w.budget)
        for h in heads:
            where = f"seq {s} head {h}"
            q_grp = q[c0:c1, h * G:(h + 1) * G]
            # stage 1: cosine of each token to the mean query
            c_gpu = r["qcos"][h, c0:c1].astype(np.float64)
            if c1 > c0:
                _, _, c_or = oracle.query_cosines(q_grp)
                err = np.max(np.abs(c_gpu - c_or))
                assert err <= QCOS_TOL, f"{where}: qcos error {err:.3g}"
            # stage 2: kept queries
            qi = r["q_idx"][s, h]
            assert np.all(qi[nq_eff:] == -1), f"{where}: q_idx padding"
            S_gpu = qi[:nq_eff].astype(np.int64)
            if c1 > c0:
                _rule_check(S_gpu, oracle.lowest_cosine_queries(c_gpu, w.n_q), c_gpu,
                            np.sort(c_gpu)[nq_eff - 1], 2 * QCOS_TOL, f"{where} q_idx")
                S_or = oracle.lowest_cosine_queries(c_or, w.n_q)
                bound = np.sort(c_or)[nq_eff - 1]
                ties["q"] += _band_check(S_gpu, S_or, c_or, bound, SEL_REL_BAND * abs(bound),
                                         f"{where} q_idx")
            # stage 3: key scores, oracle on the GPU's kept queries
            s_gpu = r["scores"][h, h0:h1].astype(np.float64)
            s_or = oracle.key_scores(q_grp[S_gpu], kh[h0:h1, h])
            if h1 > h0:
                err = np.max(np.abs(s_gpu - s_or))
                # the scorer's proven bound, on which the selections' exactness rests
                # (the errors observed are 10-20 times smaller)
                bound = score_bound(w.dtype, w.head_dim)
                assert err <= bound, f"{where}: score error {err:.3g} (bound {bound:.3g})"
            # stage 4: kept keys
            si = r["sel_idx"][s, h]
            assert np.all(si[b_eff:] == -1), f"{where}: sel_idx padding"
            I_gpu = si[:b_eff].astype(np.int64)
            if h1 > h0:
                eps = score_bound(w.dtype, w.head_dim)
                _rule_check(I_gpu, oracle.top_b_keys(s_gpu, w.budget), s_gpu,
                            np.sort(s_gpu)[::-1][b_eff - 1], 2 * eps, f"{where} sel_idx")
                I_or = oracle.top_b_keys(s_or, w.budget)
                sb = np.sort(s_or)[::-1][b_eff - 1]
                ties["k"] += _band_check(I_gpu, I_or, s_or, sb, SEL_REL_BAND * abs(sb),
                                         f"{where} sel_idx")
    return ties


def check_gather(w, r, heads=None, seqs=None):
    """K5 is a copy: bit-exact."""
    heads = range(w.num_kv_heads) if heads is None else heads
    seqs = range(w.num_seqs) if seqs is None else seqs
    for s in seqs:
        h0 = int(w.cu_hist[s])
        for h in heads:
            idx = r["sel_idx"][s, h]
            ok = idx >= 0
            for name, src in (("k_sel", w.k_hist), ("v_sel", w.v_hist)):
                got = r[name][s, h]
                want = np.zeros_like(got)
                want[ok] = src[h0 + idx[ok], h]
                assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32)), \
                    f"{name} seq {s} head {h}"


def check_attention(w, r, heads=None, seqs=None, rows=None, rng=None):
    """Attention against the oracle evaluated on the GPU's kept keys.

    rows: None = every query row; an int = that many sampled (token, head)
    rows per (sequence, KV head)."""
    q = w.q.astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    scale = 1.0 / math.sqrt(w.head_dim)
    heads = range(w.num_kv_heads) if heads is None else heads
    seqs = range(w.num_seqs) if seqs is None else seqs
    rng = rng or np.random.default_rng(0)
    worst = 0.0
    for s in seqs:
        c0, c1 = int(w.cu_chunk[s]), int(w.cu_chunk[s + 1])
        h0 = int(w.cu_hist[s])
        if c1 == c0:
            continue
        for h in heads:
            idx = r["sel_idx"][s, h]
            idx = idx[idx >= 0]
            ks = w.k_hist[h0 + idx, h]
            vs = w.v_hist[h0 + idx, h]
            kc, vc = w.k_chunk[c0:c1, h], w.v_chunk[c0:c1, h]
            if rows is None:
                for j in range(h * G, (h + 1) * G):
                    want = oracle.attend_chunk(q[c0:c1, j], ks, vs, kc, vc, scale)
                    got = r["out"][c0:c1, j].astype(np.float64)
                    worst = max(worst, float(np.max(np.abs(got - want))))
            else:
                toks = rng.integers(0, c1 - c0, size=rows)
                js = rng.integers(h * G, (h + 1) * G, size=rows)
                want = oracle.attend_rows(q[c0 + toks, js], toks, ks, vs, kc, vc, scale)
                got = r["out"][c0 + toks, js].astype(np.float64)
                worst = max(worst, float(np.max(np.abs(got - want))))
    assert worst <= ATTN_TOL[w.dtype], f"attention max-abs error {worst:.3g}"
    return worst


def check_invariants(w, r):
    """Properties that hold at any size, for every (sequence, KV head)."""
    for s in range(w.num_seqs):
        C = int(w.cu_chunk[s + 1] - w.cu_chunk[s])
        L = int(w.cu_hist[s + 1] - w.cu_hist[s])
        nq_eff, b_eff = oracle.effective_budgets(C, L, w.n_q, w.budget)
        for h in range(w.num_kv_heads):
            qi = r["q_idx"][s, h]
            si = r["sel_idx"][s, h]
            assert np.all(np.diff(qi[:nq_eff]) > 0) and np.all(qi[nq_eff:] == -1)
            assert np.all(np.diff(si[:b_eff]) > 0) and np.all(si[b_eff:] == -1)
            if nq_eff:
                assert 0 <= qi[0] and qi[nq_eff - 1] < C
            if b_eff:
                assert 0 <= si[0] and si[b_eff - 1] < L
    assert np.all(np.isfinite(r["out"]))


def check_needles(w, r):
    """Needles aligned with a kept query must be kept. Returns (hit, total, in_S)."""
    hit = in_s = 0
    for s, h, pos, tok in w.needles.tolist():
        kept_q = set(r["q_idx"][s, h].tolist())
        kept_k = set(r["sel_idx"][s, h].tolist())
        if tok in kept_q:
            in_s += 1
            assert pos in kept_k, f"needle seq {s} head {h} key {pos} (token {tok}) missed"
        hit += pos in kept_k
    return hit, len(w.needles), in_s


def run_variant(w, shape, t, variant):
    """Selection by a baseline, with every optional output."""
    sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, w.budget, want_q_idx=True,
                     want_qcos=True, want_scores=True, variant=variant)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in sel.items() if v is not None}


def check_variant_selection(w, r, variant):
    """A baseline's selection, stage-conditioned as check_selection.

    Kept queries: per-head cosines as QUOKA (none for mean_query, whose q_idx
    is all -1); for global, the oracle's head-averaged cosines and one subset
    shared by every head. Scores: the oracle's baseline scores on the GPU's
    kept queries (dot products: error bound relative to |qbar| |k|). Kept keys:
    the top-B rule on the GPU's scores, bit-exact, and the oracle's within the
    tie band. Returns tie counts."""
    q = w.q.astype(np.float64)
    kh = w.k_hist.astype(np.float64)
    Hkv = w.num_kv_heads
    G = w.num_q_heads // Hkv
    ties = {"q": 0, "k": 0}
    for s in range(w.num_seqs):
        c0, c1 = int(w.cu_chunk[s]), int(w.cu_chunk[s + 1])
        h0, h1 = int(w.cu_hist[s]), int(w.cu_hist[s + 1])
        nq_eff, b_eff = oracle.effective_budgets(c1 - c0, h1 - h0, w.n_q, w.budget)
        if variant == "global" and c1 > c0:
            cg_or = oracle.global_query_cosines(q[c0:c1], Hkv)
            S_glob = oracle.lowest_cosine_queries(cg_or, w.n_q)
        for h in range(Hkv):
            where = f"{variant} seq {s} head {h}"
            q_grp = q[c0:c1, h * G:(h + 1) * G]
            qi = r["q_idx"][s, h]
            if variant == "mean_query":
                assert np.all(qi == -1), f"{where}: q_idx must be all -1"
                S_gpu = np.arange(c1 - c0)
            else:
                assert np.all(qi[nq_eff:] == -1), f"{where}: q_idx padding"
                S_gpu = qi[:nq_eff].astype(np.int64)
                c_gpu = r["qcos"][h, c0:c1].astype(np.float64)
                if c1 > c0:
                    _, _, c_or = oracle.query_cosines(q_grp)
                    err = np.max(np.abs(c_gpu - c_or))
                    assert err <= QCOS_TOL, f"{where}: qcos error {err:.3g}"
                if variant == "global":
                    assert np.array_equal(qi, r["q_idx"][s, 0]), f"{where}: subset not shared"
                    if c1 > c0:
                        bound = np.sort(cg_or)[nq_eff - 1]
                        ties["q"] += _band_check(S_gpu, S_glob, cg_or, bound,
                                                 SEL_REL_BAND * abs(bound), f"{where} q_idx")
                elif c1 > c0:
                    _rule_check(S_gpu, oracle.lowest_cosine_queries(c_gpu, w.n_q), c_gpu,
                                np.sort(c_gpu)[nq_eff - 1], 2 * QCOS_TOL, f"{where} q_idx")
                    S_or = oracle.lowest_cosine_queries(c_or, w.n_q)
                    bound = np.sort(c_or)[nq_eff - 1]
                    ties["q"] += _band_check(S_gpu, S_or, c_or, bound, SEL_REL_BAND * abs(bound),
                                             f"{where} q_idx")
            s_gpu = r["scores"][h, h0:h1].astype(np.float64)
            k_h = kh[h0:h1, h]
            tol = np.full(h1 - h0, score_bound(w.dtype, w.head_dim, G,
                                               per_head=variant == "per_head"))
            if variant == "dot":
                s_or = oracle.key_scores(q_grp[S_gpu], k_h, sim="dot")
                if c1 > c0 and h1 > h0:
                    qbar = np.max(np.linalg.norm(q_grp[S_gpu].mean(axis=1), axis=-1))
                    tol = 1e-5 * qbar * np.linalg.norm(k_h, axis=-1) + 1e-6
            elif variant in ("mean_queries", "mean_query"):
                s_or = oracle.key_scores(q_grp[S_gpu], k_h, query_agg="mean")
            else:
                s_or = oracle.key_scores(q_grp[S_gpu], k_h)
            if h1 > h0:
                err = np.abs(s_gpu - s_or)
                assert np.all(err <= tol), \
                    f"{where}: score error {np.max(err):.3g} (bound {np.min(tol):.3g}..)"
            si = r["sel_idx"][s, h]
            assert np.all(si[b_eff:] == -1), f"{where}: sel_idx padding"
            I_gpu = si[:b_eff].astype(np.int64)
            if h1 > h0:
                rule = oracle.top_b_keys(s_gpu, w.budget)
                I_or = oracle.top_b_keys(s_or, w.budget)
                sb = np.sort(s_or)[::-1][b_eff - 1]
                if variant == "dot":
                    # unbounded dot products: no fp64 re-score, the fp32 rule decides, and
                    # the oracle's set is matched within the scores' own error
                    _rule_check(I_gpu, rule, s_gpu, 0.0, -1.0, f"{where} sel_idx")
                    band = max(SEL_REL_BAND * abs(sb), 2 * float(np.max(tol)))
                else:
                    eps = score_bound(w.dtype, w.head_dim, G, per_head=variant == "per_head")
                    _rule_check(I_gpu, rule, s_gpu, np.sort(s_gpu)[::-1][b_eff - 1], 2 * eps,
                                f"{where} sel_idx")
                    band = SEL_REL_BAND * abs(sb)
                ties["k"] += _band_check(I_gpu, I_or, s_or, sb, band, f"{where} sel_idx")
    return ties
