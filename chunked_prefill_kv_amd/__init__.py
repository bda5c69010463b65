"""Python binding of libquoka (QUOKA per-chunk hot path on MI355X / gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory and the current stream. There is no
CPU fallback: without the built library every call raises.

Entry points mirror include/quoka.h: select, gather, chunk_attn,
prefill_chunk, workspace_bytes. A `Shape` describes a batch of ragged
sequences once (it keeps the host and device prefix offsets alive).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libquoka.so")

QUOKA_OK, QUOKA_EINVAL, QUOKA_EUNSUPPORTED, QUOKA_EWORKSPACE, QUOKA_EHIP, QUOKA_ECHECK = range(6)
QUOKA_F32, QUOKA_BF16 = 0, 1
# quoka_attn_kernel values and the kernel functions they name
ATTN_KERNELS = {0: "attn_valu_kernel", 1: "attn_mfma_kernel", 2: "attn_mfma_kernel",
                3: "attn_mfma_kernel", 4: "attn_r16_kernel"}


def attn_plan(shape: Shape, kv_budget: int):
    """(quoka_attn_kernel value, key ranges) of the attention launched for this shape."""
    lib = load_library()
    k, n = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib.quoka_attn_plan(ctypes.byref(shape.c), kv_budget, ctypes.byref(k), ctypes.byref(n)),
           "quoka_attn_plan")
    return int(k.value), int(n.value)


MAX_Q_BUDGET = 128
# quoka_variant: QUOKA and the baseline selections the pages compare it with
VARIANTS = {"quoka": 0, "dot": 1, "mean_queries": 2, "mean_query": 3, "per_head": 4,
            "global": 5}

SYMBOLS = ("quoka_workspace_bytes", "quoka_select", "quoka_select_profiled",
           "quoka_select_variant", "quoka_gather", "quoka_check_selection",
           "quoka_attn_workspace_bytes", "quoka_attn_plan", "quoka_chunk_attn",
           "quoka_chunk_attn_gather", "quoka_prefill_chunk", "quoka_prefill_chunk_static",
           "quoka_prompt_workspace_bytes",
           "quoka_prefill_prompt", "quoka_strerror", "quoka_last_error")


class QuokaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({detail})")


class _CPrompt(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("prompt_len", ctypes.c_int32),
        ("chunk_len", ctypes.c_int32),
    ]


class _CShape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("cu_chunk", ctypes.c_void_p),
        ("cu_hist", ctypes.c_void_p),
        ("cu_chunk_host", ctypes.c_void_p),
        ("cu_hist_host", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libquoka.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m chunked_prefill_kv_amd.build` "
            "(the QUOKA path has no CPU fallback)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    sp = P(_CShape)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.quoka_workspace_bytes.argtypes = [sp, i32, i32, P(sz)]
    lib.quoka_select.argtypes = [sp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.quoka_select_variant.argtypes = [sp, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.quoka_select_profiled.argtypes = [sp, vp, vp, i32, i32, vp, vp, sz, vp, vp]
    lib.quoka_gather.argtypes = [sp, vp, vp, vp, i32, vp, vp, vp]
    lib.quoka_check_selection.argtypes = [sp, vp, i32, vp]
    lib.quoka_attn_workspace_bytes.argtypes = [sp, i32, P(sz)]
    lib.quoka_attn_plan.argtypes = [sp, i32, P(i32), P(i32)]
    lib.quoka_chunk_attn.argtypes = [sp, vp, vp, vp, i32, vp, vp, ctypes.c_float, vp, vp, sz, vp]
    lib.quoka_chunk_attn_gather.argtypes = [sp, vp, vp, vp, vp, i32, vp, vp, ctypes.c_float, vp,
                                            vp, sz, vp]
    lib.quoka_prefill_chunk.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_float, vp,
                                        vp, vp, sz, vp]
    lib.quoka_prefill_chunk_static.argtypes = [sp, vp, vp, vp, vp, vp, i32, i32,
                                               ctypes.c_float, vp, vp, vp]
    pp = ctypes.POINTER(_CPrompt)
    lib.quoka_prompt_workspace_bytes.argtypes = [pp, i32, i32, P(sz)]
    lib.quoka_prefill_prompt.argtypes = [pp, vp, vp, vp, i32, i32, ctypes.c_float, vp, vp, vp,
                                         sz, vp]
    for f in ("quoka_workspace_bytes", "quoka_select", "quoka_select_profiled",
              "quoka_select_variant", "quoka_gather", "quoka_check_selection", "quoka_chunk_attn",
              "quoka_chunk_attn_gather", "quoka_prefill_chunk", "quoka_prefill_chunk_static",
              "quoka_prompt_workspace_bytes", "quoka_prefill_prompt"):
        getattr(lib, f).restype = ctypes.c_int
    lib.quoka_strerror.argtypes = [ctypes.c_int]
    lib.quoka_strerror.restype = ctypes.c_char_p
    lib.quoka_last_error.argtypes = []
    lib.quoka_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != QUOKA_OK:
        lib = load_library()
        detail = lib.quoka_last_error().decode() or lib.quoka_strerror(status).decode()
        raise QuokaError(status, where, detail)


def _dtype_code(dt) -> int:
    if dt in (torch.bfloat16, "bf16"):
        return QUOKA_BF16
    if dt in (torch.float32, "fp32"):
        return QUOKA_F32
    raise ValueError(f"unsupported dtype {dt}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


class Shape:
    """Batch description: ragged chunk / history lengths and head layout.

    cu_chunk, cu_hist: prefix offsets [S + 1] (host sequences or CPU tensors).
    Device copies are made once on `device`.
    """

    def __init__(self, cu_chunk: Sequence[int], cu_hist: Sequence[int], num_q_heads: int,
                 num_kv_heads: int, head_dim: int, dtype, device="cuda"):
        self.cu_chunk_host = np.ascontiguousarray(np.asarray(cu_chunk, dtype=np.int32))
        self.cu_hist_host = np.ascontiguousarray(np.asarray(cu_hist, dtype=np.int32))
        if self.cu_chunk_host.shape != self.cu_hist_host.shape or self.cu_chunk_host.ndim != 1:
            raise ValueError("cu_chunk and cu_hist must both be [S + 1]")
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.num_seqs = int(self.cu_chunk_host.shape[0] - 1)
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.dtype_code = _dtype_code(dtype)
        self.torch_dtype = torch.bfloat16 if self.dtype_code == QUOKA_BF16 else torch.float32
        if self.device.type == "cuda":
            self.cu_chunk = torch.from_numpy(self.cu_chunk_host).to(self.device)
            self.cu_hist = torch.from_numpy(self.cu_hist_host).to(self.device)
            dev_chunk, dev_hist = self.cu_chunk.data_ptr(), self.cu_hist.data_ptr()
        else:  # host-only shapes: validation and workspace sizing, nothing runs
            self.cu_chunk = self.cu_hist = None
            dev_chunk, dev_hist = (self.cu_chunk_host.ctypes.data,
                                   self.cu_hist_host.ctypes.data)
        self.c = _CShape(self.num_seqs, num_q_heads, num_kv_heads, head_dim, self.dtype_code,
                         dev_chunk, dev_hist, self.cu_chunk_host.ctypes.data,
                         self.cu_hist_host.ctypes.data)

    @property
    def total_chunk(self) -> int:
        return int(self.cu_chunk_host[-1])

    @property
    def total_hist(self) -> int:
        return int(self.cu_hist_host[-1])

    def _check_tensor(self, t: torch.Tensor, name: str, shape, dtype=None):
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, expected {self.device}")
        if dtype is not None and t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_bytes(shape: Shape, q_budget: int, kv_budget: int) -> int:
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.quoka_workspace_bytes(ctypes.byref(shape.c), q_budget, kv_budget,
                                     ctypes.byref(n)), "quoka_workspace_bytes")
    return int(n.value)


def attn_workspace_bytes(shape: Shape, kv_budget: int) -> int:
    """Workspace bytes chunk_attn / chunk_attn_gather need (0 for most shapes)."""
    lib = load_library()
    n = ctypes.c_size_t(0)
    _check(lib.quoka_attn_workspace_bytes(ctypes.byref(shape.c), kv_budget, ctypes.byref(n)),
           "quoka_attn_workspace_bytes")
    return int(n.value)


def _attn_workspace(shape: Shape, kv_budget: int, workspace):
    if workspace is None:
        n = attn_workspace_bytes(shape, kv_budget)
        workspace = torch.empty(n, dtype=torch.uint8, device=shape.device) if n else None
    if workspace is None:
        return None, 0
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return workspace, workspace.numel()


def alloc_workspace(shape: Shape, q_budget: int, kv_budget: int) -> torch.Tensor:
    return torch.empty(workspace_bytes(shape, q_budget, kv_budget), dtype=torch.uint8,
                       device=shape.device)


def select(shape: Shape, q, k_hist, q_budget: int, kv_budget: int, *, sel_idx=None,
           want_q_idx=False, want_qcos=False, want_scores=False, workspace=None,
           variant: str = "quoka"):
    """Kept history indices per (sequence, KV head); optional stage outputs.

    ``variant`` other than "quoka" runs a baseline selection
    (quoka_select_variant; names as in VARIANTS)."""
    lib = load_library()
    if variant not in VARIANTS:
        raise ValueError(f"variant {variant!r} is not one of {sorted(VARIANTS)}")
    S, Hq, Hkv, d = shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    shape._check_tensor(q, "q", (shape.total_chunk, Hq, d), shape.torch_dtype)
    shape._check_tensor(k_hist, "k_hist", (shape.total_hist, Hkv, d), shape.torch_dtype)
    dev = shape.device
    if sel_idx is None:
        sel_idx = torch.empty((S, Hkv, kv_budget), dtype=torch.int32, device=dev)
    shape._check_tensor(sel_idx, "sel_idx", (S, Hkv, kv_budget), torch.int32)
    q_idx = torch.empty((S, Hkv, q_budget), dtype=torch.int32, device=dev) if want_q_idx else None
    qcos = torch.empty((Hkv, shape.total_chunk), dtype=torch.float32, device=dev) \
        if want_qcos else None
    scores = torch.empty((Hkv, shape.total_hist), dtype=torch.float32, device=dev) \
        if want_scores else None
    if workspace is None:
        workspace = alloc_workspace(shape, q_budget, kv_budget)
    if variant == "quoka":
        _check(lib.quoka_select(ctypes.byref(shape.c), _ptr(q), _ptr(k_hist), q_budget,
                                kv_budget, _ptr(sel_idx), _ptr(q_idx), _ptr(qcos), _ptr(scores),
                                _ptr(workspace), workspace.numel(), _stream(dev)),
               "quoka_select")
    else:
        _check(lib.quoka_select_variant(ctypes.byref(shape.c), VARIANTS[variant], _ptr(q),
                                        _ptr(k_hist), q_budget, kv_budget, _ptr(sel_idx),
                                        _ptr(q_idx), _ptr(qcos), _ptr(scores), _ptr(workspace),
                                        workspace.numel(), _stream(dev)),
               "quoka_select_variant")
    return {"sel_idx": sel_idx, "q_idx": q_idx, "qcos": qcos, "scores": scores}


def select_profiled(shape: Shape, q, k_hist, q_budget: int, kv_budget: int, sel_idx, workspace,
                    events):
    """quoka_select with four torch.cuda.Event (enable_timing) recorded between its stages:
    before the query side, before the scorer, before the top-B launches and after them."""
    lib = load_library()
    S, Hq, Hkv, d = shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    shape._check_tensor(q, "q", (shape.total_chunk, Hq, d), shape.torch_dtype)
    shape._check_tensor(k_hist, "k_hist", (shape.total_hist, Hkv, d), shape.torch_dtype)
    shape._check_tensor(sel_idx, "sel_idx", (S, Hkv, kv_budget), torch.int32)
    if len(events) != 4:
        raise ValueError("four events are needed")
    for e in events:  # torch creates the HIP event on its first record
        if not e.cuda_event:
            e.record()
    handles = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
    _check(lib.quoka_select_profiled(ctypes.byref(shape.c), _ptr(q), _ptr(k_hist), q_budget,
                                     kv_budget, _ptr(sel_idx), _ptr(workspace),
                                     workspace.numel(), handles, _stream(shape.device)),
           "quoka_select_profiled")
    return sel_idx


def gather(shape: Shape, k_hist, v_hist, sel_idx, kv_budget: int, *, k_sel=None, v_sel=None):
    lib = load_library()
    S, Hkv, d = shape.num_seqs, shape.num_kv_heads, shape.head_dim
    for t, n in ((k_hist, "k_hist"), (v_hist, "v_hist")):
        shape._check_tensor(t, n, (shape.total_hist, Hkv, d), shape.torch_dtype)
    shape._check_tensor(sel_idx, "sel_idx", (S, Hkv, kv_budget), torch.int32)
    if k_sel is None:
        k_sel = torch.empty((S, Hkv, kv_budget, d), dtype=shape.torch_dtype, device=shape.device)
    if v_sel is None:
        v_sel = torch.empty((S, Hkv, kv_budget, d), dtype=shape.torch_dtype, device=shape.device)
    _check(lib.quoka_gather(ctypes.byref(shape.c), _ptr(k_hist), _ptr(v_hist), _ptr(sel_idx),
                            kv_budget, _ptr(k_sel), _ptr(v_sel), _stream(shape.device)),
           "quoka_gather")
    return k_sel, v_sel


def check_selection(shape: Shape, sel_idx, kv_budget: int):
    """Raises QuokaError (status QUOKA_ECHECK) unless every (s, h) of sel_idx
    holds B_eff strictly ascending history positions followed by -1 padding."""
    lib = load_library()
    shape._check_tensor(sel_idx, "sel_idx", (shape.num_seqs, shape.num_kv_heads, kv_budget),
                        torch.int32)
    _check(lib.quoka_check_selection(ctypes.byref(shape.c), _ptr(sel_idx), kv_budget,
                                     _stream(shape.device)), "quoka_check_selection")


def chunk_attn(shape: Shape, q, k_sel, v_sel, kv_budget: int, k_chunk, v_chunk,
               softmax_scale: float = 0.0, *, out=None, workspace=None):
    lib = load_library()
    S, Hq, Hkv, d = shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    shape._check_tensor(q, "q", (shape.total_chunk, Hq, d), shape.torch_dtype)
    for t, n in ((k_sel, "k_sel"), (v_sel, "v_sel")):
        shape._check_tensor(t, n, (S, Hkv, kv_budget, d), shape.torch_dtype)
    for t, n in ((k_chunk, "k_chunk"), (v_chunk, "v_chunk")):
        shape._check_tensor(t, n, (shape.total_chunk, Hkv, d), shape.torch_dtype)
    if out is None:
        out = torch.empty_like(q)
    shape._check_tensor(out, "out", tuple(q.shape), shape.torch_dtype)
    ws, nws = _attn_workspace(shape, kv_budget, workspace)
    _check(lib.quoka_chunk_attn(ctypes.byref(shape.c), _ptr(q), _ptr(k_sel), _ptr(v_sel),
                                kv_budget, _ptr(k_chunk), _ptr(v_chunk), float(softmax_scale),
                                _ptr(out), _ptr(ws), nws, _stream(shape.device)),
           "quoka_chunk_attn")
    return out


def chunk_attn_gather(shape: Shape, q, k_hist, v_hist, sel_idx, kv_budget: int, k_chunk,
                      v_chunk, softmax_scale: float = 0.0, *, out=None, workspace=None):
    """Gather fused into the chunk attention: equals gather() then chunk_attn()."""
    lib = load_library()
    S, Hq, Hkv, d = shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    shape._check_tensor(q, "q", (shape.total_chunk, Hq, d), shape.torch_dtype)
    for t, n in ((k_hist, "k_hist"), (v_hist, "v_hist")):
        shape._check_tensor(t, n, (shape.total_hist, Hkv, d), shape.torch_dtype)
    shape._check_tensor(sel_idx, "sel_idx", (S, Hkv, kv_budget), torch.int32)
    for t, n in ((k_chunk, "k_chunk"), (v_chunk, "v_chunk")):
        shape._check_tensor(t, n, (shape.total_chunk, Hkv, d), shape.torch_dtype)
    if out is None:
        out = torch.empty_like(q)
    shape._check_tensor(out, "out", tuple(q.shape), shape.torch_dtype)
    ws, nws = _attn_workspace(shape, kv_budget, workspace)
    _check(lib.quoka_chunk_attn_gather(ctypes.byref(shape.c), _ptr(q), _ptr(k_hist),
                                       _ptr(v_hist), _ptr(sel_idx), kv_budget, _ptr(k_chunk),
                                       _ptr(v_chunk), float(softmax_scale), _ptr(out), _ptr(ws),
                                       nws, _stream(shape.device)), "quoka_chunk_attn_gather")
    return out


def prefill_chunk(shape: Shape, q, k_hist, v_hist, k_chunk, v_chunk, q_budget: int,
                  kv_budget: int, softmax_scale: float = 0.0, *, out=None, sel_idx=None,
                  workspace=None):
    lib = load_library()
    S, Hq, Hkv, d = shape.num_seqs, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    shape._check_tensor(q, "q", (shape.total_chunk, Hq, d), shape.torch_dtype)
    for t, n in ((k_hist, "k_hist"), (v_hist, "v_hist")):
        shape._check_tensor(t, n, (shape.total_hist, Hkv, d), shape.torch_dtype)
    for t, n in ((k_chunk, "k_chunk"), (v_chunk, "v_chunk")):
        shape._check_tensor(t, n, (shape.total_chunk, Hkv, d), shape.torch_dtype)
    if out is None:
        out = torch.empty_like(q)
    shape._check_tensor(out, "out", tuple(q.shape), shape.torch_dtype)
    if sel_idx is not None:
        shape._check_tensor(sel_idx, "sel_idx", (S, Hkv, kv_budget), torch.int32)
    if workspace is None:
        workspace = alloc_workspace(shape, q_budget, kv_budget)
    _check(lib.quoka_prefill_chunk(ctypes.byref(shape.c), _ptr(q), _ptr(k_hist), _ptr(v_hist),
                                   _ptr(k_chunk), _ptr(v_chunk), q_budget, kv_budget,
                                   float(softmax_scale), _ptr(out), _ptr(sel_idx),
                                   _ptr(workspace), workspace.numel(), _stream(shape.device)),
           "quoka_prefill_chunk")
    return out


def prefill_prompt(q, k, v, chunk_len: int, q_budget: int, kv_budget: int,
                   softmax_scale: float = 0.0, *, out=None, sel_idx=None, workspace=None):
    """Chunked prefill of one sequence's whole prompt (quoka_prefill_prompt).

    q [T, H_q, d]; k, v [T, H_kv, d] on one GPU, bf16 or fp32. sel_idx, if given, receives
    [ceil(T / chunk_len), H_kv, kv_budget] int32 (each chunk's kept history positions)."""
    lib = load_library()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, heads, d]")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q has dtype {q.dtype}; bf16 or fp32 expected")
    for t, n, h in ((k, "k", Hkv), (v, "v", Hkv)):
        if tuple(t.shape) != (T, h, d) or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{n} must be [{T}, {h}, {d}] {q.dtype} on {q.device}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous CUDA tensor")
    pr = _CPrompt(Hq, Hkv, d, QUOKA_BF16 if q.dtype == torch.bfloat16 else QUOKA_F32, T,
                  chunk_len)
    if out is None:
        out = torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    nch = -(-T // chunk_len)
    if sel_idx is not None and (tuple(sel_idx.shape) != (nch, Hkv, kv_budget)
                                or sel_idx.dtype != torch.int32 or not sel_idx.is_contiguous()):
        raise ValueError(f"sel_idx must be a contiguous int32 [{nch}, {Hkv}, {kv_budget}]")
    if workspace is None:
        n = ctypes.c_size_t(0)
        _check(lib.quoka_prompt_workspace_bytes(ctypes.byref(pr), q_budget, kv_budget,
                                                ctypes.byref(n)), "quoka_prompt_workspace_bytes")
        workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
    _check(lib.quoka_prefill_prompt(ctypes.byref(pr), _ptr(q), _ptr(k), _ptr(v), q_budget,
                                    kv_budget, float(softmax_scale), _ptr(out), _ptr(sel_idx),
                                    _ptr(workspace), workspace.numel(), _stream(q.device)),
           "quoka_prefill_prompt")
    return out
