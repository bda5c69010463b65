"""Seeded random shapes through the whole path, against the oracle.

The hand-picked cases elsewhere aim at known tile boundaries; these draw the
batch layout at random (empty and one-token chunks, empty and short
histories, GQA groups from 1 to 8 including ones that do not divide a
128-row tile, both head sizes, both dtypes, budgets from 1 to past the data)
so that a combination nobody thought of still meets the same bar: kept sets
exact within the stated bands, the layout invariants, every attention row of
one (sequence, KV head) and sampled rows of the rest within the attention
tolerance, and the fused gather bit-identical to gather + attend. The first
shapes also go through each baseline selection the pages compare against. A
few large shapes (chunks up to 4096 tokens, histories up to 64K keys, bf16)
reach the launch modes only large batches take: eight-wave attention
workgroups in the paired and the contiguous orders, and scorer tiles of up to
2048 keys. Two limit shapes: a chunk longer than the cosines the query select
holds on chip, and a 600K-key history.
"""
import numpy as np
import pytest

import chunked_prefill_kv_amd as cpk
from workloads import make_case

from gpu_check import (check_attention, check_invariants, check_selection,
                       check_variant_selection, run_stages, run_variant, upload)

pytestmark = pytest.mark.gpu

N_CASES = 40
N_VARIANT_CASES = 12
N_LARGE_CASES = 6


def per_head_fits(nq, g, d, dt):
    """The per-head baseline's on-chip limits (quoka.h): at most 640 padded
    kept rows x group, and its rows plus a 2048-bin histogram in 160 KB of LDS."""
    pad = -(-nq // 16) * 16
    rows = pad if dt == "bf16" else nq
    return pad * g <= 640 and rows * g * d * 4 + 8192 <= 160 * 1024


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    S = int(rng.integers(1, 6))
    seqs = []
    for _ in range(S):
        u = rng.random()
        C = 0 if u < 0.1 else 1 if u < 0.2 else int(rng.integers(2, 701))
        L = 0 if rng.random() < 0.1 else int(rng.integers(1, 6001))
        seqs.append((C, L))
    if sum(c for c, _ in seqs) == 0:
        seqs[0] = (int(rng.integers(1, 300)), seqs[0][1])
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 5, 7, 8]))
    d = int(rng.choice([64, 128]))
    dt = "fp32" if rng.random() < 0.3 else "bf16"
    nq = int(rng.integers(1, 129))
    b = int(rng.integers(1, 1501))
    scaled = bool(rng.random() < 0.5)
    return seqs, hkv * g, hkv, d, dt, nq, b, scaled


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    seqs, hq, hkv, d, dt, nq, b, scaled = _draw(i)
    name = f"sweep{i}"
    print(f"[gpu] {name}: seqs={seqs} Hq={hq} Hkv={hkv} d={d} {dt} Nq={nq} B={b} "
          f"scaled={scaled}", flush=True)
    w = make_case(seqs, hq, hkv, d, dt, nq, b, seed=4000 + i, scaled=scaled, name=name)
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    check_selection(w, r)
    s_full = next(s for s, (c, _) in enumerate(seqs) if c > 0)
    full = check_attention(w, r, heads=[hkv - 1], seqs=[s_full])
    err = check_attention(w, r, rows=16, rng=np.random.default_rng(i))
    assert np.array_equal(r["out_fused"], r["out"])
    print(f"[gpu] {name}: attention max-abs {full:.3g} (all rows of one head), "
          f"{err:.3g} (sampled)", flush=True)


@pytest.mark.parametrize("variant", [v for v in cpk.VARIANTS if v != "quoka"])
@pytest.mark.parametrize("i", range(N_VARIANT_CASES))
def test_random_shape_baselines(i, variant):
    seqs, hq, hkv, d, dt, nq, b, scaled = _draw(i)
    name = f"sweep{i}"
    print(f"[gpu] {name} {variant}", flush=True)
    w = make_case(seqs, hq, hkv, d, dt, nq, b, seed=4000 + i, scaled=scaled, name=name)
    shape, t = upload(w)
    if variant == "per_head" and not per_head_fits(nq, hq // hkv, d, dt):
        with pytest.raises(cpk.QuokaError) as e:
            run_variant(w, shape, t, variant)
        assert e.value.status == cpk.QUOKA_EUNSUPPORTED
        return
    r = run_variant(w, shape, t, variant)
    check_variant_selection(w, r, variant)


def _draw_large(i):
    rng = np.random.default_rng(9500 + i)
    S = int(rng.integers(1, 5))
    seqs = [(int(rng.integers(1, 4097)), int(rng.integers(0, 65537))) for _ in range(S)]
    hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 7, 8]))
    d = int(rng.choice([64, 128]))
    nq = int(rng.integers(1, 129))
    b = int(rng.integers(1, 4097))
    return seqs, hkv * g, hkv, d, "bf16", nq, b, bool(rng.random() < 0.5)


@pytest.mark.parametrize("i", range(N_LARGE_CASES))
def test_random_large_shape(i):
    seqs, hq, hkv, d, dt, nq, b, scaled = _draw_large(i)
    name = f"large{i}"
    print(f"[gpu] {name}: seqs={seqs} Hq={hq} Hkv={hkv} d={d} {dt} Nq={nq} B={b} "
          f"scaled={scaled}", flush=True)
    w = make_case(seqs, hq, hkv, d, dt, nq, b, seed=5000 + i, scaled=scaled, name=name)
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    check_selection(w, r)
    err = check_attention(w, r, rows=48, rng=np.random.default_rng(i))
    assert np.array_equal(r["out_fused"], r["out"])
    print(f"[gpu] {name}: attention max-abs {err:.3g} (sampled)", flush=True)


LIMIT_CASES = {
    # a chunk longer than the 12288 cosines the query select stages on chip
    # (it then reads them from the workspace), with the maximum query budget
    "chunk_past_lds": ([(13000, 3000)], 4, 1, 64, "bf16", 128, 512),
    # a 600K-key history: hundreds of scorer and top-B tiles per head
    "history_600k": ([(64, 600000)], 8, 2, 128, "bf16", 16, 4096),
}


@pytest.mark.parametrize("name", sorted(LIMIT_CASES))
def test_limit_shape(name):
    seqs, hq, hkv, d, dt, nq, b = LIMIT_CASES[name]
    print(f"[gpu] {name}: seqs={seqs} Hq={hq} Hkv={hkv} d={d} {dt} Nq={nq} B={b}", flush=True)
    w = make_case(seqs, hq, hkv, d, dt, nq, b, seed=6000, name=name)
    shape, t = upload(w)
    r = run_stages(w, shape, t)
    check_invariants(w, r)
    check_selection(w, r)
    err = check_attention(w, r, rows=64, rng=np.random.default_rng(1))
    assert np.array_equal(r["out_fused"], r["out"])
    print(f"[gpu] {name}: attention max-abs {err:.3g} (sampled)", flush=True)
