"""Calls on two streams at once (the header's promise: calls on different
streams may run concurrently when they share no output or workspace).

Two different batches, each with its own workspace and outputs, are issued
alternately on two streams of default priority, several times over, with no
synchronization between the streams; each stream's results must equal the
same call run alone.
"""
import pytest
import torch

import chunked_prefill_kv_amd as cpk
from workloads import make_case

from gpu_check import upload

pytestmark = pytest.mark.gpu


def test_two_streams_concurrently():
    cases = [make_case([(300, 5000), (129, 2049), (1, 700)], 8, 2, 128, "bf16", 20, 256,
                       seed=901, name="s0", scaled=True),
             make_case([(1, 3000), (1, 1500), (1, 4096)], 32, 8, 128, "bf16", 1, 1024,
                       seed=902, name="s1")]
    print("[gpu] two streams", flush=True)
    runs = []
    for w in cases:
        shape, t = upload(w)
        ws = cpk.alloc_workspace(shape, w.n_q, w.budget)
        out = torch.empty_like(t["q"])
        sel = torch.empty((w.num_seqs, w.num_kv_heads, w.budget), dtype=torch.int32,
                          device="cuda")
        call = (lambda shape=shape, t=t, ws=ws, w=w, out=out, sel=sel: cpk.prefill_chunk(
            shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"], t["v_chunk"], w.n_q,
            w.budget, out=out, sel_idx=sel, workspace=ws))
        call()
        torch.cuda.synchronize()
        runs.append((call, out, sel, out.clone(), sel.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for _, out, sel, _, _ in runs:
            out.fill_(7.0)
            sel.fill_(-7)
        torch.cuda.synchronize()
        for _ in range(4):  # interleaved issue, no cross-stream ordering
            for (call, *_), st in zip(runs, streams):
                with torch.cuda.stream(st):
                    call()
        torch.cuda.synchronize()
        for i, (_, out, sel, want_out, want_sel) in enumerate(runs):
            assert torch.equal(sel, want_sel), f"stream {i}, round {rep}: kept indices differ"
            assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), \
                f"stream {i}, round {rep}: output differs"
