"""The allocation-free entry point (quoka_prefill_chunk_static), called through
the C ABI, against quoka_prefill_chunk with a caller workspace: the same
kernels, so the same bits. Two calls in a row, the second with a smaller
problem, so the second runs on the scratch the first left behind; and a
problem beyond the static scratch is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import chunked_prefill_kv_amd as cpk
from workloads import make_case

from gpu_check import upload

pytestmark = pytest.mark.gpu


def _static(lib, w, shape, t, out, sel):
    return lib.quoka_prefill_chunk_static(
        ctypes.byref(shape.c), t["q"].data_ptr(), t["k_hist"].data_ptr(),
        t["v_hist"].data_ptr(), t["k_chunk"].data_ptr(), t["v_chunk"].data_ptr(), w.n_q,
        w.budget, ctypes.c_float(0.0), out.data_ptr(), sel.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def test_static_scratch_entry_matches_the_workspace_entry():
    lib = cpk.load_library()
    cases = [
        make_case([(300, 5000), (129, 2049), (64, 0), (1, 700)], 8, 2, 128, "bf16", 20, 256,
                  seed=611, name="static_large", scaled=True),
        make_case([(96, 1500), (33, 700)], 8, 2, 128, "bf16", 16, 128, seed=612,
                  name="static_small"),
    ]
    for w in cases:
        print(f"[gpu] static scratch entry: {w.name}", flush=True)
        shape, t = upload(w)
        S, Hkv, B = w.num_seqs, w.num_kv_heads, w.budget
        out_s = torch.empty_like(t["q"])
        sel_s = torch.empty((S, Hkv, B), dtype=torch.int32, device="cuda")
        assert _static(lib, w, shape, t, out_s, sel_s) == cpk.QUOKA_OK, \
            lib.quoka_last_error().decode()
        sel_w = torch.empty_like(sel_s)
        out_w = cpk.prefill_chunk(shape, t["q"], t["k_hist"], t["v_hist"], t["k_chunk"],
                                  t["v_chunk"], w.n_q, B, sel_idx=sel_w)
        torch.cuda.synchronize()
        assert torch.equal(sel_s, sel_w), f"{w.name}: kept indices differ"
        assert torch.equal(out_s.view(torch.int16), out_w.view(torch.int16)), \
            f"{w.name}: outputs differ"


def test_static_scratch_entry_refuses_what_does_not_fit():
    lib = cpk.load_library()
    # workspace above the static scratch: 8 KV heads of a 900k-key history
    cu_chunk, cu_hist = [0, 16], [0, 900000]
    shape = cpk.Shape(cu_chunk, cu_hist, 8, 8, 128, "bf16", device="cpu")
    need = cpk.workspace_bytes(shape, 16, 512)
    assert need > (64 << 20)
    dummy = ctypes.c_void_p(16)  # never dereferenced: the call fails before any launch
    st = lib.quoka_prefill_chunk_static(ctypes.byref(shape.c), dummy, dummy, dummy, dummy,
                                        dummy, 16, 512, ctypes.c_float(0.0), dummy, None, None)
    assert st == cpk.QUOKA_EUNSUPPORTED
    assert b"static scratch" in lib.quoka_last_error()
