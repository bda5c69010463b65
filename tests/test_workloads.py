"""Seeded input generators: determinism, bf16 rounding, shapes, needles."""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_case, make_config, round_to_bf16, bf16_bits


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                  -1.0 - 2 ** -8], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_to_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    bits = bf16_bits(got)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back, got)
    with pytest.raises(ValueError):
        bf16_bits(np.array([1.0 + 2 ** -20], np.float32))


def test_generator_is_deterministic():
    a = make_case([(33, 70), (5, 0), (17, 129)], 8, 2, 64, "bf16", 5, 40, seed=11,
                  scaled=True, needles_per_head=3)
    b = make_case([(33, 70), (5, 0), (17, 129)], 8, 2, 64, "bf16", 5, 40, seed=11,
                  scaled=True, needles_per_head=3)
    for f in ("q", "k_hist", "v_hist", "k_chunk", "v_chunk", "needles"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = make_case([(33, 70), (5, 0), (17, 129)], 8, 2, 64, "bf16", 5, 40, seed=12)
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (55, 8, 64) and a.k_hist.shape == (199, 2, 64)
    assert a.cu_chunk.tolist() == [0, 33, 38, 55] and a.cu_hist.tolist() == [0, 70, 70, 199]
    # bf16 workloads hold bf16-representable values only
    assert not np.any(a.k_hist.view(np.uint32) & 0xFFFF)
    assert a.needles.shape == (2 * 2 * 3, 4)   # the L=0 sequence gets none


def test_tiny_config_shape_and_needles():
    w = make_config("tiny")
    assert (w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim) == ("fp32", 1, 1, 64)
    assert w.chunk_lens == [128] and w.hist_lens == [1024]
    assert (w.n_q, w.budget) == (16, 128)
    assert w.needles.shape == (8, 4)
    assert len(set(w.needles[:, 2].tolist())) == 8


def test_tiny_needles_in_kept_set_are_recovered():
    """Needles aligned with a query the subselection keeps must be selected."""
    w = make_config("tiny")
    r = oracle.prefill_chunk(w.q, w.k_hist, w.v_hist, w.k_chunk, w.v_chunk,
                             w.cu_chunk, w.cu_hist, 1, w.n_q, w.budget,
                             attention=False)
    kept = set(r["q_idx"][0, 0].tolist())
    sel = set(r["sel_idx"][0, 0].tolist())
    for s, h, pos, tok in w.needles.tolist():
        if tok in kept:
            assert pos in sel


def test_outlier_needles_are_kept_and_recovered():
    """With the crowd recipe the needle queries disagree with the mean, so the
    subselection keeps them and their needles must be selected."""
    w = make_case([(96, 700), (40, 300)], 8, 2, 64, "fp32", 8, 48, seed=5,
                  needles_per_head=4, outlier_needles=6.0)
    r = oracle.prefill_chunk(w.q, w.k_hist, w.v_hist, w.k_chunk, w.v_chunk,
                             w.cu_chunk, w.cu_hist, 2, w.n_q, w.budget,
                             attention=False)
    for s, h, pos, tok in w.needles.tolist():
        assert tok in r["q_idx"][s, h].tolist()
        assert pos in r["sel_idx"][s, h].tolist()


def test_llama8b_config_shape():
    w = make_config("llama8b")
    assert w.q.shape == (2048, 32, 128) and w.k_hist.shape == (32768, 8, 128)
    assert (w.n_q, w.budget) == (64, 2048)
    # channel scales are shared by a KV head's keys and its query heads
    sd_k = w.k_hist[:, 0, :].std(axis=0)
    sd_q = w.q[:, 0:4, :].reshape(-1, 128).std(axis=0)
    assert np.corrcoef(sd_k, sd_q)[0, 1] > 0.95
    assert 0.4 < sd_k.min() and sd_k.max() < 4.5
