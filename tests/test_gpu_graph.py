"""The per-chunk path captured into a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream) and replayed.

Every launch of quoka_prefill_chunk is a kernel: counters and histograms are
cleared by the query-prep kernel, not by a memset, and nothing synchronizes
or allocates. A serving loop can therefore capture one chunk step once and
replay it. Each replay here follows eager work on the same buffers and a
synchronization, and must give the eager result bit for bit; a replay after
new inputs are copied into the captured buffers must give the eager result
on those inputs. The decode shape (one token per sequence, the attention
split into key ranges and merged) is the launch-bound case such loops have.
"""
import pytest
import torch

import chunked_prefill_kv_amd as cpk
from workloads import make_case

from gpu_check import upload

pytestmark = pytest.mark.gpu

CASES = {
    "ragged": ([(300, 5000), (129, 2049), (64, 0), (1, 700)], 8, 2, 128, 20, 256),
    "decode": ([(1, 3000), (1, 1500), (1, 0), (1, 4096)], 32, 8, 128, 1, 1024),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_chunk_replays_in_a_graph(name):
    seqs, hq, hkv, d, nq, b = CASES[name]
    print(f"[gpu] graph replay {name}", flush=True)
    w = make_case(seqs, hq, hkv, d, "bf16", nq, b, seed=811, name=name, scaled=True)
    shape, t = upload(w)
    ws = cpk.alloc_workspace(shape, nq, b)
    out = torch.empty_like(t["q"])
    sel = torch.empty((w.num_seqs, hkv, b), dtype=torch.int32, device="cuda")

    def call(o=out, s=sel):
        cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"], t["v_chunk"],
                          nq, b, out=o, sel_idx=s, workspace=ws)

    call()
    torch.cuda.synchronize()
    want_out, want_sel = out.clone(), sel.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()

    for rep in range(4):
        out.fill_(7.0)
        sel.fill_(-7)
        ws.fill_(0xA5)  # the workspace's contents on entry must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, want_sel), f"{name}: replay {rep} kept indices differ"
        assert torch.equal(out.view(torch.int16), want_out.view(torch.int16)), \
            f"{name}: replay {rep} output differs"

    # new inputs in the captured buffers
    w2 = make_case(seqs, hq, hkv, d, "bf16", nq, b, seed=812, name=name + "_2", scaled=True)
    _, t2 = upload(w2)
    for k in t:
        t[k].copy_(t2[k])
    out_e = torch.empty_like(out)
    sel_e = torch.empty_like(sel)
    call(out_e, sel_e)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_e), f"{name}: replay on new inputs, kept indices differ"
    assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), \
        f"{name}: replay on new inputs, output differs"
