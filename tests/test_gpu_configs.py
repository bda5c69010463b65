"""GPU parity at the five layer shapes' full sizes (and the decode step),
through the same entry points and launch configuration the benchmark times
(quoka_select and quoka_chunk_attn_gather; quoka_prefill_chunk must give the
same bits).

Selection: every (sequence, KV head) against the fp64 oracle, stage by stage,
with the stated tolerance (members may differ from the oracle's only within
1e-5 relative of the boundary value). Gather: every kept row, bit-exact.
Attention: every row of one KV head per shape against the oracle evaluated on
the GPU's kept keys, and sampled rows of every other KV head. Properties that
hold at any size (ordering, padding, finiteness, needles kept) everywhere.
"""
import functools

import numpy as np
import pytest
import torch

import chunked_prefill_kv_amd as cpk
from workloads import make_config

from gpu_check import (upload, run_stages, check_selection, check_gather, check_attention,
                       check_invariants, check_needles)

pytestmark = pytest.mark.gpu

# shape -> KV head whose attention rows are all checked (the other heads: sampled rows)
FULL_HEAD = {"llama8b": 3, "narrow": 1, "ragged": 5, "long": 6, "decode": 2}
SAMPLED_ROWS = 16
NAMES = ["llama8b", "narrow", "ragged", "long", "decode"]


@functools.lru_cache(maxsize=1)
def _run(name):
    print(f"[gpu] config {name}: generating", flush=True)
    w = make_config(name)
    shape, t = upload(w)
    print(f"[gpu] config {name}: running", flush=True)
    r = run_stages(w, shape, t)
    sel = torch.empty((w.num_seqs, w.num_kv_heads, w.budget), dtype=torch.int32, device="cuda")
    out = cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"],
                            t["v_chunk"], w.n_q, w.budget, sel_idx=sel)
    torch.cuda.synchronize()
    same = (np.array_equal(sel.cpu().numpy(), r["sel_idx"]) and
            np.array_equal(out.float().cpu().numpy(), r["out"]))
    del t, out, sel
    torch.cuda.empty_cache()
    return w, r, same


@pytest.mark.parametrize("name,part", [(n, p) for n in NAMES for p in ("select", "attend")])
def test_config_parity(name, part):
    w, r, same = _run(name)
    if part == "select":
        assert same, "quoka_prefill_chunk differs from the stage-wise calls"
        check_invariants(w, r)
        print(f"[gpu] config {name}: oracle selection of all {w.num_seqs} x {w.num_kv_heads} "
              "(sequence, KV head) pairs", flush=True)
        ties = check_selection(w, r)
        check_gather(w, r)
        msg = f"[gpu] config {name}: ties {ties}"
        if w.needles.shape[0]:
            hit, total, in_s = check_needles(w, r)
            msg += f", needles kept {hit}/{total} ({in_s} aligned with kept queries)"
        print(msg, flush=True)
    else:
        h = FULL_HEAD[name]
        print(f"[gpu] config {name}: every attention row of KV head {h}", flush=True)
        full = check_attention(w, r, heads=[h])
        others = [x for x in range(w.num_kv_heads) if x != h]
        samp = check_attention(w, r, heads=others, rows=SAMPLED_ROWS,
                               rng=np.random.default_rng(7))
        print(f"[gpu] config {name}: attention max-abs {full:.3g} (all rows of head {h}), "
              f"{samp:.3g} (sampled rows of the others)", flush=True)
