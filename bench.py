"""Throughput of QUOKA's per-chunk hot path on one MI355X.

A step is one pass of the whole path (query subselection, key scoring, top-B
select, K/V gather, chunk attention) over one layer's chunk, all heads, with
inputs already resident in HBM. By default the gather runs fused into the
attention (quoka_select, then quoka_chunk_attn_gather); --unfused times the
three separate calls (quoka_select, quoka_gather, quoka_chunk_attn); --variant
times one of the pages' baseline selections in place of QUOKA's (then without
the CPU baseline). Rotated copies of every input, at least 1 GiB of them in
all, are cycled through, so a step finds none of its bytes in the 256 MB
last-level cache.

Prints ONE JSON line. `value` comes from a timed pass of the steps alone; a
second timed pass brackets every stage with HIP events on the stream the
kernels run on (they cost the stream ~10 us per step, so they are kept out of
the first pass) and gives the stage times and the roofline entry for the
dominant kernel (chunk attention, bf16 MFMA). cpu_baseline times the fp64
oracle on a bounded sample of the same workload on the host cores.

usage: python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--config long]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 (vector / MFMA)
PEAK_HBM_GBS = 8000.0

DESCR = {
    "tiny": "1 seq, 1q/1kv heads, d=64, fp32, L=1024, C=128, Nq=16, B=128",
    "llama8b": "Llama-3-8B-shaped layer: 1 seq, 32q/8kv heads, d=128, bf16, L=32768, C=2048, "
               "Nq=64, B=2048",
    "long": "long-history layer: 1 seq, 32q/8kv heads, d=128, bf16, L=131072, C=4096, Nq=128, "
            "B=4096",
    "narrow": "narrow-GQA layer: 1 seq, 28q/4kv heads, d=128, bf16, L=65536, C=1024, Nq=32, "
              "B=1024",
    "ragged": "8 ragged seqs, L=4K..96K, C=512 each, 32q/8kv heads, d=128, bf16, Nq=32, B=1024",
    "decode": "decode step: 8 seqs, C=1 each, L=16384, 32q/8kv heads, d=128, bf16, Nq=1, B=2048",
}


def attention_flops(w) -> float:
    """Algorithmic FLOPs of the chunk attention: 4 d H_q per visible (query, key) pair,
    pairs = sum_s C_s B_eff + C_s (C_s + 1) / 2."""
    pairs = 0
    for C, L in zip(w.chunk_lens, w.hist_lens):
        pairs += C * min(w.budget, L) + C * (C + 1) // 2
    return 4.0 * w.head_dim * w.num_q_heads * pairs


def _elem(w) -> int:
    return 2 if w.dtype == "bf16" else 4


def scorer_bytes(w) -> float:
    """Algorithmic HBM bytes of the scorer: every history key once, plus the scores."""
    return w.k_hist.shape[0] * w.num_kv_heads * (w.head_dim * _elem(w) + 4)


def attention_bytes(w) -> float:
    """Algorithmic HBM bytes of the chunk attention: Q, the B_eff kept K/V rows per (sequence,
    KV head) and the chunk's K/V read once, O written once."""
    tc = int(w.cu_chunk[-1])
    kept = sum(min(w.budget, int(L)) for L in w.hist_lens) * w.num_kv_heads
    return _elem(w) * w.head_dim * (2 * tc * w.num_q_heads + 2 * kept + 2 * tc * w.num_kv_heads)


def gather_bytes(w) -> float:
    """Algorithmic HBM bytes of the gather: the selected K and V rows read, K/V_sel written
    (padding rows past B_eff are written only), plus the indices."""
    sel = sum(min(w.budget, int(L)) for L in w.hist_lens) * w.num_kv_heads
    rows = w.num_seqs * w.num_kv_heads * w.budget
    return _elem(w) * w.head_dim * 2 * (sel + rows) + 4 * rows


def attention_kernel_name(w) -> str:
    """The attention kernel the library launches for this layer (quoka_attn_plan)."""
    import chunked_prefill_kv_amd as cpk
    shape = cpk.Shape(w.cu_chunk, w.cu_hist, w.num_q_heads, w.num_kv_heads, w.head_dim,
                      w.dtype, device="cpu")
    return cpk.ATTN_KERNELS[cpk.attn_plan(shape, w.budget)[0]]


def measured_traffic(config: str, kernel: str, source: str):
    """HBM bytes per launch from the committed counter runs (profiles/hbm_traffic.md), or
    None when they are missing or the kernel source changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        text = open(path).read()
        block = text[text.index("```json") + 7:]
        data = json.loads(block[:block.index("```")])
        rec = data[config][kernel]
        csrc = os.path.join(ROOT, "chunked_prefill_kv_amd", "csrc")
        for f, want in ((source, rec["source"]["sha256_16"]),
                        ("common.h", rec["source"]["common.h"])):
            got = hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()[:16]
            if got != want:
                return None
        return float(rec["hbm_bytes"])
    except (OSError, ValueError, KeyError):
        return None


def cpu_baseline(w, min_seconds: float = 10.0, max_runs: int = 5):
    """The fp64 oracle over the whole layer (every KV head and its query heads: selection
    and attention), repeated until about min_seconds of CPU work; median run time."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    times = []
    t_all = time.perf_counter()
    while len(times) < max_runs and (not times or time.perf_counter() - t_all < min_seconds):
        t0 = time.perf_counter()
        oracle.prefill_chunk(w.q, w.k_hist, w.v_hist, w.k_chunk, w.v_chunk, w.cu_chunk,
                             w.cu_hist, w.num_kv_heads, w.n_q, w.budget)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {
        "value": float(w.cu_chunk[-1]) / med,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle, whole path for the whole layer (all {w.num_kv_heads} KV "
                   f"heads, {w.num_q_heads} query heads), {len(times)} runs, median {med:.2f} s, "
                   f"total {sum(times):.1f} s; host has {cores} cores, BLAS used {threads} "
                   f"threads, the rest of the oracle runs on one"),
    }


def bench_peaks():
    """Measured peaks next to the published ones the rooflines divide by: a loop of
    independent v_mfma_f32_32x32x16_bf16 on every SIMD (two waves each), a streaming
    16-byte read of 4 GiB, a 2 GiB device copy, and the shader cycle counter against the
    100 MHz real-time counter."""
    import ctypes
    import torch
    from chunked_prefill_kv_amd import build as cbuild
    if not os.path.exists(cbuild.PEAKS_LIB):
        raise RuntimeError(f"{cbuild.PEAKS_LIB} is missing: build it first")
    lib = ctypes.CDLL(cbuild.PEAKS_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.quoka_peaks_mfma.argtypes = [i32, i32, vp, vp]
    lib.quoka_peaks_read.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
    lib.quoka_peaks_clock.argtypes = [i32, vp, vp, vp]
    lib.quoka_peaks_device.argtypes = [ctypes.POINTER(i32)] * 4
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    st = torch.cuda.current_stream().cuda_stream
    info = [ctypes.c_int(0) for _ in range(4)]
    assert lib.quoka_peaks_device(*[ctypes.byref(x) for x in info]) == 0
    clock_khz, mem_khz, bus_bits, cus = (x.value for x in info)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3  # seconds

    blocks, iters = cus * 2, 20000  # two four-wave workgroups per CU: two waves per SIMD
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    t = timed(lambda: lib.quoka_peaks_mfma(blocks, iters, sink.data_ptr(), st), 3)
    mfma_tflops = blocks * 4 * iters * 4 * 32768 / t / 1e12
    buf = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    rblocks = cus * 16
    rsink = torch.empty(rblocks * 256, dtype=torch.float32, device=dev)
    t = timed(lambda: lib.quoka_peaks_read(buf.data_ptr(), buf.numel(), rblocks,
                                           rsink.data_ptr(), st), 5)
    read_gbs = buf.numel() / t / 1e9
    src = buf[: 2 << 30]
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), 5)
    copy_gbs = 2 * src.numel() / t / 1e9
    del buf, dst
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    csink = torch.empty(64, dtype=torch.float32, device=dev)
    assert lib.quoka_peaks_clock(1 << 22, cnt.data_ptr(), csink.data_ptr(), st) == 0
    torch.cuda.synchronize()
    t0, t1, r0, r1 = (int(x) for x in cnt.cpu())
    memtime_mhz = (t1 - t0) / ((r1 - r0) / 100e6) / 1e6 if r1 > r0 else None
    # dense bf16: 1024 flop per clock per SIMD, four SIMDs per CU
    mfma_clock_mhz = mfma_tflops * 1e12 / (cus * 4 * 1024) / 1e6
    print(json.dumps({
        "probe": "peaks", "cus": cus, "clock_rate_attr_MHz": clock_khz / 1e3,
        "memory_clock_attr_MHz": mem_khz / 1e3, "memory_bus_bits": bus_bits,
        "mfma_bf16_dense_TFLOPs": round(mfma_tflops, 1),
        "mfma_frac_of_published_2500": round(mfma_tflops / PEAK_BF16_TFLOPS, 3),
        "mfma_implied_clock_MHz": round(mfma_clock_mhz, 1),
        "hbm_read_GBps": round(read_gbs, 1), "hbm_copy_GBps": round(copy_gbs, 1),
        "hbm_read_frac_of_published_8000": round(read_gbs / PEAK_HBM_GBS, 3),
        "shader_counter_MHz": None if memtime_mhz is None else round(memtime_mhz, 1),
    }), flush=True)


def bench_prompt(args):
    """Whole-prompt chunked prefill of one sequence (llama8b heads: 32/8, d=128, bf16,
    N_q=64, B=2048): quoka_prefill_prompt against dense chunked prefill, where every chunk
    attends to its whole history (the same attention kernel with every history key kept)."""
    import torch
    import chunked_prefill_kv_amd as cpk
    T, Bc, Hq, Hkv, d, nq, B = args.prompt, args.chunk, 32, 8, 128, 64, 2048
    g = torch.Generator(device="cuda").manual_seed(20260100)
    q = torch.randn(T, Hq, d, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(T, Hkv, d, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(T, Hkv, d, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty_like(q)
    nch = -(-T // Bc)
    ws = None

    def quoka():
        nonlocal ws
        if ws is None:
            import ctypes
            pr = cpk._CPrompt(Hq, Hkv, d, cpk.QUOKA_BF16, T, Bc)
            sz = ctypes.c_size_t(0)
            cpk.load_library().quoka_prompt_workspace_bytes(ctypes.byref(pr), nq, B,
                                                            ctypes.byref(sz))
            ws = torch.empty(sz.value, dtype=torch.uint8, device="cuda")
        cpk.prefill_prompt(q, k, v, Bc, nq, B, out=out, workspace=ws)

    dense_calls = []
    for i in range(nch):
        a, b = i * Bc, min(T, (i + 1) * Bc)
        shape = cpk.Shape([0, b - a], [0, a], Hq, Hkv, d, "bf16")
        kb = max(a, 1)
        idx = torch.arange(kb, dtype=torch.int32, device="cuda")
        if a == 0:
            idx.fill_(-1)
        idx = idx.view(1, 1, kb).expand(1, Hkv, kb).contiguous()
        dense_calls.append((shape, a, b, kb, idx))
    # the attention's own workspace (key-range states of short chunks), allocated once
    dense_ws = torch.empty(max([cpk.attn_workspace_bytes(c[0], c[3]) for c in dense_calls] + [16]),
                           dtype=torch.uint8, device="cuda")

    def dense():
        for shape, a, b, kb, idx in dense_calls:
            cpk.chunk_attn_gather(shape, q[a:b], k[:a], v[:a], idx, kb, k[a:b], v[a:b],
                                  out=out[a:b], workspace=dense_ws)

    res = {}
    for name, fn in (("quoka", quoka), ("dense", dense)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / args.steps
    line = {
        "metric": "whole-prompt chunked prefill tokens/s (one layer, QUOKA selection per chunk)",
        "value": T / (res["quoka"] * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["quoka"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v)",
        "config": {"workload": f"prompt of {T} tokens in chunks of {Bc}, 32q/8kv heads, d=128, "
                               f"bf16, Nq={nq}, B={B}", "chunks": nch},
        "dense": {"ms_per_prompt": res["dense"], "tokens_per_s": T / (res["dense"] * 1e-3),
                  "what": "every chunk attends to its whole history (no selection)"},
        "speedup_vs_dense": res["dense"] / res["quoka"],
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first; the first few tens of steps after start run "
                         "slower (the clocks settle), so the default is 50")
    ap.add_argument("--config", default="long", choices=sorted(DESCR))
    ap.add_argument("--input-sets", type=int, default=0,
                    help="rotated copies of the inputs cycled through (default: enough for "
                         "1 GiB, four times the 256 MB last-level cache, at least 2)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="gather into K/V_sel and attend in separate calls")
    ap.add_argument("--prompt", type=int, default=0, metavar="T",
                    help="time a whole prompt of T tokens through chunked prefill "
                         "(quoka_prefill_prompt) against dense chunked prefill instead")
    ap.add_argument("--chunk", type=int, default=2048, help="chunk length for --prompt")
    ap.add_argument("--variant", default="quoka",
                    choices=["quoka", "dot", "mean_queries", "mean_query", "per_head", "global"],
                    help="time a baseline selection (quoka_select_variant) in place of QUOKA's")
    ap.add_argument("--peaks", action="store_true",
                    help="only confirm the chip's peaks (dense bf16 MFMA loop, HBM streaming "
                         "read and copy, shader clock) and print them as one JSON line")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times) and exit: the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is built "
              "for a single MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_prefill_kv_amd as cpk
    from workloads import make_config

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)
        return

    if args.peaks:
        bench_peaks()
        return

    if args.prompt:
        bench_prompt(args)
        return

    w = make_config(args.config)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = cpk.Shape(w.cu_chunk, w.cu_hist, w.num_q_heads, w.num_kv_heads, w.head_dim,
                      w.dtype, device=dev)
    names = ("q", "k_hist", "v_hist", "k_chunk", "v_chunk")
    base = {n: torch.from_numpy(getattr(w, n)).to(dt).to(dev) for n in names}
    # Rotated copies of every input (the same work on different bytes): a step
    # finds nothing the previous steps left in the 256 MB last-level cache, so
    # the bytes the kernels read come from HBM.
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    nsets = args.input_sets or min(16, max(2, -(-(1 << 30) // set_bytes)))
    sets = [base]
    TL = w.k_hist.shape[0]
    TC = w.q.shape[0]
    for r in range(1, nsets):
        sets.append({n: torch.roll(base[n], (r * (TL if "hist" in n else TC)) // nsets, 0)
                     .contiguous() for n in names})
    S, Hkv, B = w.num_seqs, w.num_kv_heads, w.budget
    ws = cpk.alloc_workspace(shape, w.n_q, B)
    sel = torch.empty((S, Hkv, B), dtype=torch.int32, device=dev)
    k_sel = v_sel = None
    if args.unfused:
        k_sel = torch.empty((S, Hkv, B, w.head_dim), dtype=dt, device=dev)
        v_sel = torch.empty_like(k_sel)
    out = torch.empty_like(base["q"])

    # ev (second pass): 0 before the selection, 1 before its scorer, 2 before its top-B,
    # 3 after the selection, 4 after the gather, 5 after the attention
    def step(i, ev=None):
        x = sets[i % len(sets)]
        if ev is not None and args.variant == "quoka":
            cpk.select_profiled(shape, x["q"], x["k_hist"], w.n_q, B, sel, ws, ev[0:4])
        else:
            if ev is not None:
                ev[0].record()
            cpk.select(shape, x["q"], x["k_hist"], w.n_q, B, sel_idx=sel, workspace=ws,
                       variant=args.variant)
            if ev is not None:
                for e in ev[1:4]:
                    e.record()
        if args.unfused:
            cpk.gather(shape, x["k_hist"], x["v_hist"], sel, B, k_sel=k_sel, v_sel=v_sel)
        if ev is not None:
            ev[4].record()
        if args.unfused:
            cpk.chunk_attn(shape, x["q"], k_sel, v_sel, B, x["k_chunk"], x["v_chunk"], out=out,
                           workspace=ws)
        else:
            cpk.chunk_attn_gather(shape, x["q"], x["k_hist"], x["v_hist"], sel, B, x["k_chunk"],
                                  x["v_chunk"], out=out, workspace=ws)
        if ev is not None:
            ev[5].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Two timed passes of `steps` steps each. The first times the steps alone:
    # `value` and ms_per_step. The second brackets every stage with events on
    # the stream the kernels run on, for the stage times and the roofline's
    # kernel duration; those events themselves cost the stream ~10 us per step,
    # so the step time is not taken from that pass.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + args.steps + i, evs[i])
    torch.cuda.synchronize()
    span = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in evs]) * 1e3  # noqa: E731
    per = {"select": span(0, 3), "gather": span(3, 4), "attention": span(4, 5)}
    if args.variant == "quoka":
        per.update({"select_query_side": span(0, 1), "select_scorer": span(1, 2),
                    "select_topb": span(2, 3)})
    sel_us, gat_us, att_us = (float(np.mean(per[k])) for k in ("select", "gather", "attention"))
    pct = {k: {"p10": round(float(np.percentile(v, 10)), 2),
               "p50": round(float(np.percentile(v, 50)), 2),
               "p90": round(float(np.percentile(v, 90)), 2)}
           for k, v in per.items() if args.unfused or k != "gather"}

    tokens = float(w.cu_chunk[-1])
    flops = attention_flops(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = flops / (att_us * 1e-6) / 1e12
    attn_kernel = attention_kernel_name(w)
    traffic = measured_traffic(args.config, attn_kernel, "attention.hip")
    gbytes = gather_bytes(w)
    line = {
        "metric": "chunk-prefill attn tokens/sec per layer (select+gather+attn); "
                  "HBM/MFMA % of peak",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generators, no dataset or weights)",
        "config": {"workload": f"{args.config}: {DESCR[args.config]}",
                   "chunk_tokens": int(tokens), "history_tokens": int(TL),
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "q_budget": w.n_q, "kv_budget": B,
                   "input_sets": len(sets), "selection": args.variant,
                   "path": "select + gather + chunk_attn" if args.unfused
                           else "select + chunk_attn_gather (gather fused)"},
        "stages_us_pct": pct,
        "stages_us": ({"select": round(sel_us, 2), "gather": round(gat_us, 2),
                       "chunk_attn": round(att_us, 2)} if args.unfused else
                      {"select": round(sel_us, 2), "chunk_attn_gather": round(att_us, 2)}),
        "roofline": {"bound": "mfma", "kernel": attn_kernel,
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "algorithmic": {"flops_per_launch": flops,
                                     "bytes_per_launch": attention_bytes(w)}},
        "secondary": ({"gather_GBps": gbytes / (gat_us * 1e-6) / 1e9,
                       "gather_frac_hbm": gbytes / (gat_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                       "gather_bytes": gbytes} if args.unfused else
                      {"gather": "fused into the attention (quoka_chunk_attn_gather)"}),
    }
    if args.variant == "quoka":
        sc_us = float(np.mean(per["select_scorer"]))
        sc_gbs = scorer_bytes(w) / (sc_us * 1e-6) / 1e9
        line["secondary"].update({
            "scorer_us": round(sc_us, 2), "scorer_bytes": scorer_bytes(w),
            "scorer_GBps": round(sc_gbs, 1), "scorer_frac_hbm": round(sc_gbs / PEAK_HBM_GBS, 4),
            "scorer_timing": "HIP events around the scorer launch, same run (the launch gap "
                             "included)"})
    if not args.no_cpu_baseline and args.variant == "quoka":
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
