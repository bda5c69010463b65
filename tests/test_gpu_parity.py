"""GPU parity of every stage against the fp64 oracle, at sizes the oracle
finishes in seconds (several tiles per kernel plus ragged tails), and the edge
cases: empty history, one-token chunk, budgets above the data, the largest
query budget, zero vectors, head_dim 64 and 128, GQA groups of 1, 2, 4, 7 and 8,
and decode-like batches (every chunk one or two tokens). The small bf16 cases
run the attention with each tile's keys split into ranges (a key range that
starts past some rows' tokens included) and merged; one case runs it unsplit.
"""
import math

import numpy as np
import pytest
import torch

import chunked_prefill_kv_amd as cpk
import oracle
from workloads import make_case, make_config

from gpu_check import (upload, run_stages, check_selection, check_gather, check_attention,
                       check_invariants, check_needles)

pytestmark = pytest.mark.gpu

CASES = {
    # name: (seqs [(C, L)], H_q, H_kv, d, dtype, N_q, B, extra)
    "fp32_d128_g2_ragged": ([(70, 3000), (1, 500), (33, 0), (130, 40)], 4, 2, 128, "fp32",
                            8, 64, {}),
    "fp32_d64_g1": ([(200, 2500)], 2, 2, 64, "fp32", 16, 300, {}),
    "bf16_d128_g4_ragged": ([(300, 5000), (129, 2049), (64, 0), (1, 700)], 8, 2, 128, "bf16",
                            20, 256, dict(scaled=True)),
    "bf16_d128_g7_maxq": ([(200, 4100)], 14, 2, 128, "bf16", 128, 1000, {}),
    "bf16_d64_g2": ([(100, 3000), (17, 1500)], 4, 2, 64, "bf16", 32, 300, {}),
    "bf16_d128_g1_rope": ([(150, 2000)], 2, 2, 128, "bf16", 16, 128, dict(rope_base=1e6)),
    "bf16_budget_above_data": ([(90, 50), (40, 500)], 8, 2, 128, "bf16", 200 // 2, 600, {}),
    "bf16_needles": ([(256, 3000), (128, 1500)], 8, 2, 128, "bf16", 8, 32,
                     dict(needles_per_head=4, outlier_needles=6.0)),
    # decode-like chunks (C_s * G <= 8): one partly filled 128-row attention tile per KV head
    "bf16_decode_g4": ([(1, 3000), (1, 0), (2, 500), (1, 64)], 8, 2, 128, "bf16", 1, 256, {}),
    "bf16_decode_g8": ([(1, 1500), (1, 70)], 16, 2, 128, "bf16", 2, 1000, dict(scaled=True)),
    "bf16_decode_d64_g1": ([(1, 2000), (1, 100), (1, 1)], 2, 2, 64, "bf16", 1, 300, {}),
    # 140 128-row attention tiles (between 128 and 256: at most one per CU, no
    # key split): sixteen rows per wave, eight waves per tile (at most 128
    # tiles split their keys into ranges and merge, as every smaller case here)
    "bf16_four_wave_unsplit": ([(1100, 1500)], 16, 4, 128, "bf16", 16, 200, {}),
    # scorer tiles of 1024 keys (four streamed blocks per wave), last tile partial
    "bf16_scorer_tiles_1024": ([(64, 33000)], 8, 8, 128, "bf16", 16, 512, {}),
    # scorer tiles of 512 keys: many short histories, some waves with one block
    "bf16_scorer_tiles_512": ([(2, 300)] * 270, 4, 2, 128, "bf16", 2, 128, {}),
}


def _case(name, seed=1234):
    seqs, hq, hkv, d, dt, nq, b, extra = CASES[name]
    return make_case(seqs, hq, hkv, d, dt, nq, b, seed, name=name, **extra)


@pytest.mark.parametrize("name", sorted(CASES))
def test_stage_parity(name):
    print(f"[gpu] stage parity {name}", flush=True)
    w = _case(name)
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    ties = check_selection(w, r)
    check_gather(w, r)
    err = check_attention(w, r)
    # the gather fused into the attention reads the same rows in the same order
    assert np.array_equal(r["out_fused"], r["out"]), "fused gather differs from gather + attend"
    print(f"[gpu] {name}: ties {ties}, attention max-abs {err:.3g}", flush=True)
    if w.needles.shape[0]:
        hit, total, in_s = check_needles(w, r)
        assert in_s == total  # the outlier recipe puts every needle query in the kept set


def test_fused_equals_stagewise():
    """quoka_prefill_chunk runs the same kernels: bit-identical output."""
    w = _case("bf16_d128_g4_ragged")
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    sel = torch.empty((w.num_seqs, w.num_kv_heads, w.budget), dtype=torch.int32, device="cuda")
    out = cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"],
                            t["v_chunk"], w.n_q, w.budget, sel_idx=sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), r["sel_idx"])
    assert np.array_equal(out.float().cpu().numpy(), r["out"])


def test_fused_gather_handles_padding_and_bad_indices():
    """chunk_attn_gather == gather + chunk_attn when sel_idx holds -1 padding in the middle and
    indices outside [0, L_s) (both read as zero rows), for both kernels (bf16 MFMA, fp32)."""
    for name in ("bf16_d128_g4_ragged", "fp32_d128_g2_ragged", "bf16_decode_g4"):
        print(f"[gpu] fused gather, bad indices {name}", flush=True)
        w = _case(name)
        shape, t = upload(w)
        B = w.budget
        sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, B)["sel_idx"]
        g = torch.Generator().manual_seed(7)
        mask = torch.rand(sel.shape, generator=g) < 0.2
        junk = torch.randint(-5, 10**6, sel.shape, generator=g, dtype=torch.int32)
        sel = torch.where(mask.to(sel.device), junk.to(sel.device), sel).contiguous()
        k_sel, v_sel = cpk.gather(shape, t["k_hist"], t["v_hist"], sel, B)
        out = cpk.chunk_attn(shape, t["q"], k_sel, v_sel, B, t["k_chunk"], t["v_chunk"])
        fused = cpk.chunk_attn_gather(shape, t["q"], t["k_hist"], t["v_hist"], sel, B,
                                      t["k_chunk"], t["v_chunk"])
        torch.cuda.synchronize()
        assert torch.equal(out, fused)


@pytest.mark.parametrize("name", ["bf16_d128_g7_maxq", "bf16_four_wave_unsplit"])
def test_repeat_runs_are_bitwise_identical(name):
    # key ranges merged afterwards; and sixteen rows per wave
    print(f"[gpu] repeat runs {name}", flush=True)
    w = _case(name)
    shape, t = upload(w)
    ws = cpk.alloc_workspace(shape, w.n_q, w.budget)
    outs = []
    for _ in range(10):
        sel = torch.empty((w.num_seqs, w.num_kv_heads, w.budget), dtype=torch.int32,
                          device="cuda")
        o = cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"],
                              t["v_chunk"], w.n_q, w.budget, sel_idx=sel, workspace=ws)
        torch.cuda.synchronize()
        outs.append((sel.cpu().numpy(), o.view(torch.int16).cpu().numpy()))
    for a, b in outs[1:]:
        assert np.array_equal(a, outs[0][0]) and np.array_equal(b, outs[0][1])


def test_zero_vectors():
    """Zero queries and keys: unit(0) = 0, so their cosines and scores are 0."""
    w = make_case([(96, 800)], 8, 2, 128, "bf16", 16, 64, seed=99, name="zeros")
    w.q[5] = 0.0                 # a whole token
    w.q[7, 0:4] = 0.0            # one KV group of a token
    w.k_hist[10:20, 1] = 0.0     # keys of head 1
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    check_selection(w, r)
    check_attention(w, r)
    assert np.all(r["scores"][1, 10:20] == 0.0)


def test_all_zero_chunk_keeps_lowest_tokens():
    """All-zero queries: the mean query is 0, every cosine is 0, ties keep 0..N_q-1."""
    w = make_case([(50, 300)], 4, 1, 128, "fp32", 6, 20, seed=5, name="zero_chunk")
    w.q[:] = 0.0
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    assert r["q_idx"][0, 0].tolist() == list(range(6))
    assert np.all(r["qcos"] == 0.0)
    # every score is 0 too: the first B keys are kept
    assert r["sel_idx"][0, 0].tolist() == list(range(20))


def test_tiny_config_full_parity():
    w = make_config("tiny")
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    check_selection(w, r)
    check_gather(w, r)
    check_attention(w, r)
    hit, total, in_s = check_needles(w, r)
    print(f"[gpu] tiny needles kept {hit}/{total} ({in_s} aligned with kept queries)")


def test_binding_rejects_wrong_inputs():
    w = _case("fp32_d64_g1")
    shape, t = upload(w)
    with pytest.raises(ValueError):
        cpk.select(shape, t["q"].to(torch.bfloat16), t["k_hist"], 8, 16)
    with pytest.raises(cpk.QuokaError) as e:
        cpk.select(shape, t["q"], t["k_hist"], 0, 16)
    assert e.value.status == cpk.QUOKA_EINVAL
    with pytest.raises(cpk.QuokaError) as e:
        cpk.select(shape, t["q"], t["k_hist"], 8, 16,
                   workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == cpk.QUOKA_EWORKSPACE


ORDER_CASES = {
    # eight-wave workgroups pairing a heavy and a light 128-row tile; 33 tiles
    # leave the middle one without a partner
    "pair_odd": ([(1056, 3000)], 32, 8, 128, "bf16", 16, 512),
    # the paired order over a ragged batch: the shorter chunk needs fewer pairs
    "pair_ragged": ([(1024, 2000), (500, 1500)], 32, 8, 128, "bf16", 16, 512),
    # 256 contiguous rows per workgroup; the last workgroup has one tile only
    "wide_odd": ([(1056, 600)] * 8, 32, 8, 128, "bf16", 8, 256),
    # the same two orders with head_dim 64 (K/V tiles of 8 rows per 1 KB LDS piece)
    "pair_odd_d64": ([(1056, 3000)], 32, 8, 64, "bf16", 16, 512),
    "wide_odd_d64": ([(1056, 600)] * 8, 32, 8, 64, "bf16", 8, 256),
    # four 128-row tiles: each tile's keys split into 8 ranges (mostly history),
    # merged afterwards
    "split8_history": ([(64, 8000)], 8, 2, 128, "bf16", 16, 1024),
    # 20 tiles, 6 ranges over 2..6 key tiles: ranges inside the chunk start past
    # the tokens of a tile's first rows (those rows see no key in them), and the
    # short tiles leave some ranges empty
    "split6_chunk": ([(300, 100)], 8, 2, 128, "bf16", 8, 64),
    # sixteen rows per wave (156 tiles of 128 rows, one per CU at most): GQA 7,
    # a partly filled last tile; and head_dim 64 over two sequences (152 tiles)
    "r16_g7": ([(700, 900)], 28, 4, 128, "bf16", 16, 256),
    "r16_d64": ([(600, 700), (300, 400)], 16, 4, 64, "bf16", 8, 128),
    # 560 four-wave tiles, too few for eight-wave workgroups and more than two
    # per CU: the unsplit four-wave kernel with 32 rows per wave
    "four_wave_32rows": ([(1100, 800)] * 4, 16, 4, 128, "bf16", 8, 256),
    # GQA 7: 128-row tiles cut through a token's heads (paired order, 66 tiles)
    "pair_g7": ([(1200, 3000)], 28, 4, 128, "bf16", 16, 512),
    # enough tiles for eight-wave workgroups, but a chunk of at most half the
    # kept history's key tiles: the paired order (15 tiles per problem, so one
    # middle tile without a partner), over 8 sequences
    "pair_short_chunk": ([(480, 5000)] * 8, 32, 8, 128, "bf16", 8, 1024),
    # one query head per KV head in the wide order, chunks of different lengths
    "wide_g1": ([(4096, 300), (3000, 900)] * 4, 8, 8, 128, "bf16", 8, 128),
}


@pytest.mark.parametrize("name", sorted(ORDER_CASES))
def test_attention_tile_orders(name):
    """The attention's workgroup orders (paired, wide, odd tile counts) against the oracle:
    every row of the first and last KV head of the first and last sequence (all the
    workgroups of those (sequence, KV head) pairs), sampled rows everywhere else; and the
    fused gather bit-identical to gather + attend."""
    seqs, hq, hkv, d, dt, nq, b = ORDER_CASES[name]
    print(f"[gpu] attention order {name}", flush=True)
    w = make_case(seqs, hq, hkv, d, dt, nq, b, seed=31, name=name)
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    check_selection(w, r)
    ends = sorted({0, w.num_seqs - 1})
    full = check_attention(w, r, heads=sorted({0, hkv - 1}), seqs=ends)
    err = check_attention(w, r, rows=48, rng=np.random.default_rng(5))
    assert np.array_equal(r["out_fused"], r["out"])
    print(f"[gpu] {name}: attention max-abs {full:.3g} (all rows), {err:.3g} (sampled)",
          flush=True)


def test_cosines_skipped_when_every_token_is_kept():
    """With every chunk at most q_budget tokens long the cosine pass is skipped unless the
    caller asks for the cosines; the selections are the same either way."""
    w = _case("bf16_decode_g4")
    shape, t = upload(w)
    a = cpk.select(shape, t["q"], t["k_hist"], 4, w.budget, want_q_idx=True, want_scores=True)
    b = cpk.select(shape, t["q"], t["k_hist"], 4, w.budget, want_q_idx=True, want_qcos=True,
                   want_scores=True)
    torch.cuda.synchronize()
    for k in ("sel_idx", "q_idx", "scores"):
        assert torch.equal(a[k], b[k]), k
