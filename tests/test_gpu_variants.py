"""GPU parity of the baseline selections (quoka_select_variant) against the
fp64 oracle's select_for_sequence, stage by stage, on ragged batches with an
empty history, an empty chunk, a one-token chunk, head_dim 64 and 128, fp32
and bf16 and GQA groups of 1, 2 and 4; and the whole chunk (baseline
selection, then the fused gather-attention) against the oracle's prefill.
"""
import math

import numpy as np
import pytest
import torch

import chunked_prefill_kv_amd as cpk
import oracle
from workloads import make_case

from gpu_check import (upload, run_variant, check_variant_selection, check_attention,
                       ATTN_TOL, SEL_REL_BAND)

pytestmark = pytest.mark.gpu

VARIANTS = [v for v in cpk.VARIANTS if v != "quoka"]

CASES = {
    # name: (seqs [(C, L)], H_q, H_kv, d, dtype, N_q, B, extra)
    "fp32_d128_g2": ([(70, 3000), (1, 500), (33, 0), (0, 700), (130, 40)], 4, 2, 128, "fp32",
                     8, 64, {}),
    "bf16_d128_g4": ([(300, 5000), (129, 2049), (64, 0), (1, 700)], 8, 2, 128, "bf16", 20, 256,
                     dict(scaled=True)),
    "bf16_d64_g1": ([(200, 3000), (17, 1500)], 2, 2, 64, "bf16", 32, 300, {}),
}


def _case(name, seed=4321):
    seqs, hq, hkv, d, dt, nq, b, extra = CASES[name]
    return make_case(seqs, hq, hkv, d, dt, nq, b, seed, name=name, **extra)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", sorted(CASES))
def test_variant_selection_parity(name, variant):
    w = _case(name)
    print(f"[variants] {name} {variant}", flush=True)
    shape, t = upload(w)
    r = run_variant(w, shape, t, variant)
    ties = check_variant_selection(w, r, variant)
    print(f"  ties {ties}", flush=True)


@pytest.mark.parametrize("variant", ["dot", "mean_query", "global"])
def test_variant_chunk_matches_oracle_prefill(variant):
    """Baseline selection followed by the fused gather-attention: the kept keys
    within the tie bands of the oracle's prefill_chunk, and the attention on
    the GPU's kept keys within the attention tolerance."""
    w = _case("bf16_d128_g4", seed=99)
    print(f"[variants] chunk {variant}", flush=True)
    shape, t = upload(w)
    sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, w.budget, variant=variant)
    out = cpk.chunk_attn_gather(shape, t["q"], t["k_hist"], t["v_hist"], sel["sel_idx"],
                                w.budget, t["k_chunk"], t["v_chunk"])
    torch.cuda.synchronize()
    r = {"sel_idx": sel["sel_idx"].cpu().numpy(), "out": out.float().cpu().numpy()}
    ref = oracle.prefill_chunk(w.q, w.k_hist, w.v_hist, w.k_chunk, w.v_chunk, w.cu_chunk,
                               w.cu_hist, w.num_kv_heads, w.n_q, w.budget, attention=False,
                               variant=variant)
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        h0, h1 = int(w.cu_hist[s]), int(w.cu_hist[s + 1])
        c0, c1 = int(w.cu_chunk[s]), int(w.cu_chunk[s + 1])
        b_eff = min(w.budget, h1 - h0)
        for h in range(w.num_kv_heads):
            got = r["sel_idx"][s, h][:b_eff].astype(np.int64)
            assert np.all(r["sel_idx"][s, h][b_eff:] == -1)
            want = ref["sel_idx"][s, h][:b_eff]
            if h1 == h0:
                continue
            s_or = ref["scores"][h, h0:h1]
            sb = np.sort(s_or)[::-1][b_eff - 1]
            band = SEL_REL_BAND * abs(sb)
            if variant == "dot" and c1 > c0:
                # the unbounded dot products keep their fp32 ranking: widen by their error
                q_grp = w.q[c0:c1, h * G:(h + 1) * G].astype(np.float64)
                qbar = np.max(np.linalg.norm(q_grp.mean(axis=1), axis=-1))
                kn = np.max(np.linalg.norm(w.k_hist[h0:h1, h].astype(np.float64), axis=-1))
                band = max(band, 2 * (1e-5 * qbar * kn + 1e-6))
            diff = set(got.tolist()) ^ set(want.tolist())
            bad = [i for i in diff if abs(s_or[i] - sb) > band]
            assert not bad, (variant, s, h, len(bad), bad[:5])
    check_attention(w, r, rows=32, rng=np.random.default_rng(3))


def test_per_head_scores_equal_quoka_scores():
    """Scoring each head and averaging gives QUOKA's scores up to rounding, and
    the same kept keys outside the tie band."""
    w = _case("bf16_d128_g4", seed=7)
    shape, t = upload(w)
    a = run_variant(w, shape, t, "per_head")
    b = run_variant(w, shape, t, "quoka")
    np.testing.assert_array_equal(a["q_idx"], b["q_idx"])
    np.testing.assert_allclose(a["scores"], b["scores"], atol=4e-6, rtol=0)


def test_per_head_rejects_what_does_not_fit_on_chip():
    w = make_case([(200, 1000)], 14, 2, 128, "bf16", 128, 64, 5)
    shape, t = upload(w)
    with pytest.raises(cpk.QuokaError):
        cpk.select(shape, t["q"], t["k_hist"], 128, 64, variant="per_head")
