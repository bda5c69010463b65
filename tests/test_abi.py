"""The C ABI without a GPU: the library loads, exports what include/quoka.h
declares, and validates arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import chunked_prefill_kv_amd as cpk
from chunked_prefill_kv_amd import build as cbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quoka.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(cpk.LIB_PATH):
        cbuild.build()
    return cpk.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(quoka_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(cpk.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", cpk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (quoka_\w+)", out))
    assert set(_declared()) <= exported
    for name in _declared():
        assert hasattr(lib, name)


def test_library_is_built_for_gfx950(lib):
    out = subprocess.run(["strings", cpk.LIB_PATH], capture_output=True, text=True).stdout
    assert "gfx950" in out


def _host_shape(cu_chunk, cu_hist, hq=8, hkv=2, d=128, dtype="bf16"):
    return cpk.Shape(cu_chunk, cu_hist, hq, hkv, d, dtype, device="cpu")


def _ws_status(shape, qb, kvb):
    n = ctypes.c_size_t(0)
    st = cpk.load_library().quoka_workspace_bytes(ctypes.byref(shape.c), qb, kvb,
                                                  ctypes.byref(n))
    return st, n.value


def test_workspace_size_grows_with_the_problem(lib):
    st1, n1 = _ws_status(_host_shape([0, 100], [0, 1000]), 16, 64)
    st2, n2 = _ws_status(_host_shape([0, 100, 300], [0, 1000, 5000]), 16, 64)
    st3, n3 = _ws_status(_host_shape([0, 100], [0, 1000]), 32, 512)
    assert (st1, st2, st3) == (0, 0, 0)
    assert 0 < n1 < n2 and n1 < n3
    assert n1 % 256 == 0


@pytest.mark.parametrize("kw,qb,kvb,code", [
    (dict(hq=6, hkv=4), 8, 8, cpk.QUOKA_EINVAL),          # H_q not a multiple of H_kv
    (dict(d=96), 8, 8, cpk.QUOKA_EUNSUPPORTED),           # head_dim not built
    (dict(), 0, 8, cpk.QUOKA_EINVAL),                     # q_budget < 1
    (dict(), cpk.MAX_Q_BUDGET + 1, 8, cpk.QUOKA_EUNSUPPORTED),
    (dict(), 8, 0, cpk.QUOKA_EINVAL),                     # kv_budget < 1
])
def test_workspace_validation(lib, kw, qb, kvb, code):
    st, _ = _ws_status(_host_shape([0, 10], [0, 20], **kw), qb, kvb)
    assert st == code
    assert lib.quoka_last_error().decode()
    assert lib.quoka_strerror(code).decode()


def test_every_status_has_its_own_message(lib):
    codes = (cpk.QUOKA_OK, cpk.QUOKA_EINVAL, cpk.QUOKA_EUNSUPPORTED, cpk.QUOKA_EWORKSPACE,
             cpk.QUOKA_EHIP, cpk.QUOKA_ECHECK)
    msgs = [lib.quoka_strerror(c).decode() for c in codes]
    assert len(set(msgs)) == len(codes) and "unknown status" not in msgs
    assert lib.quoka_strerror(len(codes)).decode() == "unknown status"


def test_check_selection_validates_before_any_launch(lib):
    shape = _host_shape([0, 10], [0, 20])
    assert lib.quoka_check_selection(ctypes.byref(shape.c), None, 8, None) == cpk.QUOKA_EINVAL
    assert "sel_idx" in lib.quoka_last_error().decode()
    assert lib.quoka_check_selection(ctypes.byref(shape.c), ctypes.c_void_p(16), 0,
                                     None) == cpk.QUOKA_EINVAL


def test_bad_offsets_are_rejected(lib):
    assert _ws_status(_host_shape([0, 10, 5], [0, 20, 30]), 8, 8)[0] == cpk.QUOKA_EINVAL
    assert _ws_status(_host_shape([1, 10], [0, 20]), 8, 8)[0] == cpk.QUOKA_EINVAL
    bad = _host_shape([0, 10], [0, 20])
    bad.c.num_seqs = 0
    assert _ws_status(bad, 8, 8)[0] == cpk.QUOKA_EINVAL
    bad = _host_shape([0, 10], [0, 20])
    bad.c.dtype = 7
    assert _ws_status(bad, 8, 8)[0] == cpk.QUOKA_EINVAL


def test_select_rejects_missing_workspace_before_any_launch(lib):
    shape = _host_shape([0, 10], [0, 20])
    buf = np.zeros(4096, np.uint8)  # host memory: never dereferenced
    p = buf.ctypes.data
    st = lib.quoka_select(ctypes.byref(shape.c), p, p, 4, 8, p, None, None, None, None, 0, None)
    assert st == cpk.QUOKA_EWORKSPACE
    st = lib.quoka_select(ctypes.byref(shape.c), p, p, 4, 8, p, None, None, None, p, 16, None)
    assert st == cpk.QUOKA_EWORKSPACE
    assert "needs" in lib.quoka_last_error().decode()


def test_null_and_misaligned_inputs_are_rejected(lib):
    shape = _host_shape([0, 10], [0, 20])
    buf = np.zeros(4096, np.uint8)
    p = buf.ctypes.data + (16 - buf.ctypes.data % 16) % 16
    st = lib.quoka_prefill_chunk(ctypes.byref(shape.c), None, p, p, p, p, 4, 8, 0.0, p, None, p,
                                 1 << 30, None)
    assert st == cpk.QUOKA_EINVAL and "q is null" in lib.quoka_last_error().decode()
    st = lib.quoka_chunk_attn(ctypes.byref(shape.c), p + 2, p, p, 8, p, p, 0.0, p, None, 0, None)
    assert st == cpk.QUOKA_EINVAL and "aligned" in lib.quoka_last_error().decode()
    st = lib.quoka_chunk_attn(ctypes.byref(shape.c), p, p, p, 8, p, p, float("nan"), p, None, 0, None)
    assert st == cpk.QUOKA_EINVAL
    st = lib.quoka_gather(ctypes.byref(shape.c), p, p, None, 8, p, p, None)
    assert st == cpk.QUOKA_EINVAL
    st = lib.quoka_chunk_attn_gather(ctypes.byref(shape.c), p, p, p, None, 8, p, p, 0.0, p, None, 0, None)
    assert st == cpk.QUOKA_EINVAL and "sel_idx is null" in lib.quoka_last_error().decode()
    st = lib.quoka_chunk_attn_gather(ctypes.byref(shape.c), p, p, p + 4, p, 8, p, p, 0.0, p, None, 0, None)
    assert st == cpk.QUOKA_EINVAL and "aligned" in lib.quoka_last_error().decode()


def _attn_ws(shape, kvb):
    n = ctypes.c_size_t(0)
    st = cpk.load_library().quoka_attn_workspace_bytes(ctypes.byref(shape.c), kvb, ctypes.byref(n))
    return st, n.value


def test_attention_workspace_only_for_shapes_that_split_their_keys(lib):
    # decode: 8 sequences of one token, 64 (sequence, KV head) tiles on 256 CUs
    dec = _host_shape(list(range(9)), [16384 * i for i in range(9)], hq=32, hkv=8)
    st, n = _attn_ws(dec, 2048)
    # four key ranges: 8 * 32 rows, 4 * 128 + 8 bytes each per range
    assert st == 0 and n == 4 * 8 * 32 * (4 * 128 + 8)
    # a 2048-token chunk with 8 KV heads fills the chip: no split, no workspace
    big = _host_shape([0, 2048], [0, 32768], hq=32, hkv=8)
    assert _attn_ws(big, 2048) == (0, 0)
    # fp32 runs the VALU kernel, which never splits
    assert _attn_ws(_host_shape(list(range(9)), [16384 * i for i in range(9)], hq=32, hkv=8,
                                dtype="fp32"), 2048) == (0, 0)
    # the per-chunk workspace covers the attention's states as well
    st, nsel = _ws_status(dec, 1, 2048)
    assert st == 0 and nsel >= n


def test_split_attention_without_workspace_is_rejected(lib):
    shape = _host_shape(list(range(9)), [16384 * i for i in range(9)], hq=32, hkv=8)
    buf = np.zeros(4096, np.uint8)
    p = buf.ctypes.data + (16 - buf.ctypes.data % 16) % 16
    st = lib.quoka_chunk_attn(ctypes.byref(shape.c), p, p, p, 2048, p, p, 0.0, p, None, 0, None)
    assert st == cpk.QUOKA_EWORKSPACE and "needs" in lib.quoka_last_error().decode()
    st = lib.quoka_chunk_attn_gather(ctypes.byref(shape.c), p, p, p, p, 2048, p, p, 0.0, p, p, 64,
                                     None)
    assert st == cpk.QUOKA_EWORKSPACE and "needs" in lib.quoka_last_error().decode()


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    monkeypatch.setattr(cpk, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        cpk.load_library(str(tmp_path / "missing.so"))


@pytest.mark.parametrize("variant,cu_chunk,hq,qb,code,msg", [
    (9, [0, 10], 8, 8, cpk.QUOKA_EINVAL, "variant"),
    (-1, [0, 10], 8, 8, cpk.QUOKA_EINVAL, "variant"),
    (cpk.VARIANTS["global"], [0, 12289], 8, 8, cpk.QUOKA_EUNSUPPORTED, "cross-head"),
    (cpk.VARIANTS["per_head"], [0, 10], 14, 128, cpk.QUOKA_EUNSUPPORTED, "per-head"),
])
def test_select_variant_validation(lib, variant, cu_chunk, hq, qb, code, msg):
    """Baseline limits are checked on the host, before the workspace or any launch."""
    shape = _host_shape(cu_chunk, [0, 20], hq=hq)
    buf = np.zeros(4096, np.uint8)
    p = buf.ctypes.data + (16 - buf.ctypes.data % 16) % 16
    st = lib.quoka_select_variant(ctypes.byref(shape.c), variant, p, p, qb, 8, p, None, None,
                                  None, None, 0, None)
    assert st == code and msg in lib.quoka_last_error().decode()


def test_peak_probe_library_exports_its_probes(lib):
    """The bench's peak probes are a library of their own, outside the boundary."""
    path = cbuild.PEAKS_LIB
    if not os.path.exists(path):
        cbuild.build()
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    names = set(re.findall(r"\bT (quoka_peaks_\w+)", out))
    assert names == {"quoka_peaks_mfma", "quoka_peaks_read", "quoka_peaks_clock",
                     "quoka_peaks_device"}


def test_attention_plan_of_the_layer_shapes(lib):
    """quoka_attn_plan (host only): the kernel and key ranges each layer shape's attention
    takes, as the benchmark names them in its roofline entry."""
    ragged_hist = [0]
    for k in (4, 8, 16, 24, 32, 48, 64, 96):
        ragged_hist.append(ragged_hist[-1] + k * 1024)
    cases = {
        # name: (cu_chunk, cu_hist, H_q, H_kv, d, dtype, B) -> (kernel, key ranges)
        "tiny": (([0, 128], [0, 1024], 1, 1, 64, "fp32", 128), (0, 1)),
        "llama8b": (([0, 2048], [0, 32768], 32, 8, 128, "bf16", 2048), (3, 1)),
        "long": (([0, 4096], [0, 131072], 32, 8, 128, "bf16", 4096), (2, 1)),
        "narrow": (([0, 1024], [0, 65536], 28, 4, 128, "bf16", 1024), (4, 1)),
        "ragged": (([512 * i for i in range(9)], ragged_hist, 32, 8, 128, "bf16", 1024), (3, 1)),
        "decode": ((list(range(9)), [16384 * i for i in range(9)], 32, 8, 128, "bf16", 2048),
                   (1, 4)),
    }
    for name, ((cc, ch, hq, hkv, d, dt, b), want) in cases.items():
        shape = cpk.Shape(cc, ch, hq, hkv, d, dt, device="cpu")
        assert cpk.attn_plan(shape, b) == want, name
    k = ctypes.c_int32(0)
    shape = _host_shape([0, 100], [0, 1000])
    assert lib.quoka_attn_plan(ctypes.byref(shape.c), 64, ctypes.byref(k), None) == cpk.QUOKA_EINVAL
