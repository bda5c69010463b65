"""QUOKA_DEBUG mode and quoka_check_selection, through the C ABI.

In debug mode every entry point checks its device arguments before its first
compute kernel (offsets equal to their host copies, finite Q/K/V, kept-index
inputs in range) and the selection's output afterwards. The planted mistakes
below are all caught by those checks before any compute kernel runs, so no
kernel ever sees them; the out-of-range values are ones the kernels would in
any case read as zero rows. quoka_check_selection is tested on selections the
library wrote and on copies of them with one entry broken in each way the
layout forbids.
"""
import pytest
import torch

import chunked_prefill_kv_amd as cpk
from workloads import make_case

from gpu_check import upload

pytestmark = pytest.mark.gpu


def _case(seed=701, name="debug"):
    # ragged, with a sequence whose history is shorter than the budget (-1 padding)
    return make_case([(96, 1500), (33, 100), (64, 700)], 8, 2, 128, "bf16", 16, 128,
                     seed=seed, name=name)


def _prefill(w, shape, t):
    sel = torch.empty((w.num_seqs, w.num_kv_heads, w.budget), dtype=torch.int32, device="cuda")
    out = cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"],
                            t["v_chunk"], w.n_q, w.budget, sel_idx=sel)
    torch.cuda.synchronize()
    return out, sel


def _raises(fn, status, *words):
    with pytest.raises(cpk.QuokaError) as e:
        fn()
    torch.cuda.synchronize()
    assert e.value.status == status, str(e.value)
    for wd in words:
        assert wd in str(e.value), (wd, str(e.value))
    return str(e.value)


def test_debug_mode_gives_the_same_results(monkeypatch):
    w = _case()
    print(f"[gpu] debug mode on {w.name}", flush=True)
    shape, t = upload(w)
    out0, sel0 = _prefill(w, shape, t)
    monkeypatch.setenv("QUOKA_DEBUG", "1")
    out1, sel1 = _prefill(w, shape, t)
    assert torch.equal(sel0, sel1)
    assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
    # every stage entry point runs its checks and passes
    r = cpk.select(shape, t["q"], t["k_hist"], w.n_q, w.budget)
    assert torch.equal(r["sel_idx"], sel0)
    k_sel, v_sel = cpk.gather(shape, t["k_hist"], t["v_hist"], sel0, w.budget)
    a = cpk.chunk_attn(shape, t["q"], k_sel, v_sel, w.budget, t["k_chunk"], t["v_chunk"])
    b = cpk.chunk_attn_gather(shape, t["q"], t["k_hist"], t["v_hist"], sel0, w.budget,
                              t["k_chunk"], t["v_chunk"])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out0.view(torch.int16))
    assert torch.equal(b.view(torch.int16), out0.view(torch.int16))


def test_debug_mode_reports_non_finite_inputs(monkeypatch):
    w = _case(seed=702, name="debug_nan")
    shape, t = upload(w)
    monkeypatch.setenv("QUOKA_DEBUG", "1")
    Hq, d = w.num_q_heads, w.head_dim
    q = t["q"].clone()
    q[17, 3, 40] = float("nan")
    msg = _raises(lambda: cpk.select(shape, q, t["k_hist"], w.n_q, w.budget),
                  cpk.QUOKA_EINVAL, "q", "non-finite")
    assert f"row {17 * Hq + 3}" in msg and "element 40" in msg, msg
    kc = t["k_chunk"].clone()
    kc[5, 1, 0] = float("inf")
    _raises(lambda: cpk.chunk_attn_gather(shape, t["q"], t["k_hist"], t["v_hist"],
                                          torch.full((w.num_seqs, w.num_kv_heads, w.budget), -1,
                                                     dtype=torch.int32, device="cuda"),
                                          w.budget, kc, t["v_chunk"]),
            cpk.QUOKA_EINVAL, "k_chunk", "non-finite")
    vh = t["v_hist"].clone()
    vh[1000, 0, 127] = float("-inf")
    _raises(lambda: cpk.prefill_chunk(shape, t["q"], t["k_hist"], vh, t["k_chunk"],
                                      t["v_chunk"], w.n_q, w.budget),
            cpk.QUOKA_EINVAL, "v_hist", "non-finite", "element 127")
    # k_sel rows past B_eff are never read: a NaN there is not reported, one
    # below B_eff is (sequence 1 has a 100-key history: B_eff = 100)
    out0, sel0 = _prefill(w, shape, t)
    monkeypatch.setenv("QUOKA_DEBUG", "1")
    k_sel, v_sel = cpk.gather(shape, t["k_hist"], t["v_hist"], sel0, w.budget)
    k_sel[1, 0, 110, :] = float("nan")
    cpk.chunk_attn(shape, t["q"], k_sel, v_sel, w.budget, t["k_chunk"], t["v_chunk"])
    k_sel[1, 0, 99, 2] = float("nan")
    _raises(lambda: cpk.chunk_attn(shape, t["q"], k_sel, v_sel, w.budget, t["k_chunk"],
                                   t["v_chunk"]),
            cpk.QUOKA_EINVAL, "k_sel", "non-finite")


def test_debug_mode_reports_bad_indices_and_offsets(monkeypatch):
    w = _case(seed=703, name="debug_idx")
    shape, t = upload(w)
    _, sel = _prefill(w, shape, t)
    monkeypatch.setenv("QUOKA_DEBUG", "1")
    bad = sel.clone()
    bad[2, 1, 5] = 700  # sequence 2 has 700 history keys: positions 0..699
    _raises(lambda: cpk.gather(shape, t["k_hist"], t["v_hist"], bad, w.budget),
            cpk.QUOKA_EINVAL, "sel_idx[s=2, h=1, b=5]")
    bad = sel.clone()
    bad[0, 0, 0] = -2
    _raises(lambda: cpk.chunk_attn_gather(shape, t["q"], t["k_hist"], t["v_hist"], bad,
                                          w.budget, t["k_chunk"], t["v_chunk"]),
            cpk.QUOKA_EINVAL, "sel_idx[s=0, h=0, b=0]")
    # device offsets that disagree with the host copy (smaller, so in bounds
    # whatever happened): refused before any launch
    shape.cu_hist[1] -= 1
    _raises(lambda: cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"],
                                      t["v_chunk"], w.n_q, w.budget),
            cpk.QUOKA_EINVAL, "cu_hist[1]")


def test_check_selection_accepts_selections_and_catches_each_broken_rule():
    w = _case(seed=704, name="check_sel")
    print(f"[gpu] check_selection on {w.name}", flush=True)
    shape, t = upload(w)
    for n_q in (1, w.n_q):
        sel = cpk.select(shape, t["q"], t["k_hist"], n_q, w.budget)["sel_idx"]
        cpk.check_selection(shape, sel, w.budget)
    for variant in ("dot", "mean_query"):
        sel = cpk.select(shape, t["q"], t["k_hist"], w.n_q, w.budget,
                         variant=variant)["sel_idx"]
        cpk.check_selection(shape, sel, w.budget)
    _, sel = _prefill(w, shape, t)
    cpk.check_selection(shape, sel, w.budget)

    def broken(s, h, b, value=None, swap=False):
        x = sel.clone()
        if swap:
            x[s, h, b], x[s, h, b + 1] = sel[s, h, b + 1].item(), sel[s, h, b].item()
        else:
            x[s, h, b] = value
        return x

    cases = [
        (broken(0, 1, 10, swap=True), (0, 1, 11)),              # descending pair
        (broken(0, 0, 7, value=sel[0, 0, 6].item()), (0, 0, 7)),  # duplicate
        (broken(2, 0, 3, value=700), (2, 0, 3)),                 # past L_s (700)
        (broken(0, 1, 4, value=-1), (0, 1, 4)),                  # padding below B_eff
        (broken(1, 1, 100, value=5), (1, 1, 100)),               # no padding at B_eff = 100
        (broken(2, 1, 0, value=-5), (2, 1, 0)),                  # negative
    ]
    for x, (s, h, b) in cases:
        _raises(lambda: cpk.check_selection(shape, x, w.budget), cpk.QUOKA_ECHECK,
                f"sel_idx[s={s}, h={h}, b={b}]")
