"""Whole-prompt chunked prefill (quoka_prefill_prompt) on the GPU.

* The driver runs the per-chunk path once per chunk: its output and kept
  indices equal, bit for bit, quoka_prefill_chunk called chunk by chunk on the
  same tensors (history = all earlier tokens).
* Against the oracle's whole-prompt loop: fp32 with generic random data (no
  near-ties in either selection), selections equal and outputs within the fp32
  attention tolerance; bf16 with a budget that keeps the whole history, where
  the result is dense causal attention.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_kv_amd as cpk
import oracle

from gpu_check import ATTN_TOL

pytestmark = pytest.mark.gpu


def _prompt(T, Hq, Hkv, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, Hq, d, generator=g)
    k = torch.randn(T, Hkv, d, generator=g)
    v = torch.randn(T, Hkv, d, generator=g)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [x.to(dt).cuda().contiguous() for x in (q, k, v)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prompt_equals_chunk_by_chunk_calls(dtype):
    print(f"[gpu] prompt vs chunk calls {dtype}", flush=True)
    T, Hq, Hkv, d, Bc, nq, B = 1000, 8, 2, 128, 256, 16, 160
    q, k, v = _prompt(T, Hq, Hkv, d, dtype, 5)
    nch = -(-T // Bc)
    sel = torch.full((nch, Hkv, B), -7, dtype=torch.int32, device="cuda")
    out = cpk.prefill_prompt(q, k, v, Bc, nq, B, sel_idx=sel)
    for i in range(nch):
        a, b = i * Bc, min(T, (i + 1) * Bc)
        shape = cpk.Shape([0, b - a], [0, a], Hq, Hkv, d, dtype)
        s_i = torch.empty((1, Hkv, B), dtype=torch.int32, device="cuda")
        o_i = cpk.prefill_chunk(shape, q[a:b].contiguous(), k[:a].contiguous(),
                                v[:a].contiguous(), k[a:b].contiguous(),
                                v[a:b].contiguous(), nq, B, sel_idx=s_i)
        torch.cuda.synchronize()
        assert torch.equal(s_i[0], sel[i]), f"chunk {i}: kept indices differ"
        assert torch.equal(o_i, out[a:b]), f"chunk {i}: output differs"
    assert torch.all(sel[0] == -1)  # chunk 0 has no history


def test_prompt_matches_oracle_fp32():
    print("[gpu] prompt vs oracle fp32", flush=True)
    T, Hq, Hkv, d, Bc, nq, B = 640, 4, 2, 64, 160, 12, 100
    q, k, v = _prompt(T, Hq, Hkv, d, "fp32", 6)
    nch = -(-T // Bc)
    sel = torch.empty((nch, Hkv, B), dtype=torch.int32, device="cuda")
    out = cpk.prefill_prompt(q, k, v, Bc, nq, B, sel_idx=sel)
    torch.cuda.synchronize()
    ref = oracle.prefill_prompt(q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy(), Bc, Hkv,
                                nq, B)
    assert np.array_equal(sel.cpu().numpy(), ref["sel_idx"])
    err = np.abs(out.cpu().numpy() - ref["out"]).max()
    print(f"[gpu] prompt fp32 max-abs {err:.3g}", flush=True)
    assert err <= ATTN_TOL["fp32"]


def test_prompt_with_full_budget_is_dense_bf16():
    print("[gpu] prompt full budget bf16", flush=True)
    T, Hq, Hkv, d, Bc = 777, 8, 2, 128, 128
    q, k, v = _prompt(T, Hq, Hkv, d, "bf16", 7)
    out = cpk.prefill_prompt(q, k, v, Bc, 8, T)
    torch.cuda.synchronize()
    ref = oracle.prefill_prompt(q.float().cpu().numpy(), k.float().cpu().numpy(),
                                v.float().cpu().numpy(), Bc, Hkv, 8, T)
    err = np.abs(out.float().cpu().numpy() - ref["out"]).max()
    print(f"[gpu] prompt dense bf16 max-abs {err:.3g}", flush=True)
    assert err <= ATTN_TOL["bf16"]
