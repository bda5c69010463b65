"""Seeded generators for the five layer shapes and for small test cases.

All values are drawn in float32 from NumPy's PCG64 and, for bf16 workloads,
rounded once to bf16 (round to nearest, ties to even). The arrays returned are
float32 whose values are exactly representable in the workload's dtype, so an
fp64 up-cast on the CPU and a bf16 upload to the GPU see the same numbers.

Layouts (token-major): q [sum C, H_q, d]; k_hist, v_hist [sum L, H_kv, d];
k_chunk, v_chunk [sum C, H_kv, d]; cu_chunk, cu_hist [S + 1] int32 offsets.

Recipes (the pages fix no input distribution; these stand in for the long
context suites they evaluate on, which are not used here):
  * plain:   Q, K, V ~ N(0, 1).
  * scaled:  per KV head h a channel-scale vector sigma_h = exp(U[ln .5, ln 4])
             multiplies K (history and chunk) and the group's query heads,
             mimicking outlier channels shared by queries and keys; V ~ N(0,1).
  * rope:    rotate-half rotary embedding (base 1e6) at positions 0..L-1 for
             history keys and L..L+C-1 for chunk queries and chunk keys.
  * needles: a history key at a random position is replaced by
             3 * sqrt(d) * unit(sum_j q_{c,j}) + noise, where c is a random
             chunk token, the sum runs over the KV head's query heads and the
             noise is drawn like an ordinary key of the workload.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["CONFIGS", "Workload", "make_config", "make_case",
           "round_to_bf16", "bf16_bits"]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable float32 -> its uint16 bit pattern."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("values are not bf16-representable; round first")
    return (b >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                       # "fp32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    n_q: int                         # query budget N_q
    budget: int                      # KV budget B
    cu_chunk: np.ndarray             # int32 [S + 1]
    cu_hist: np.ndarray              # int32 [S + 1]
    q: np.ndarray                    # float32 [sum C, H_q, d]
    k_hist: np.ndarray               # float32 [sum L, H_kv, d]
    v_hist: np.ndarray
    k_chunk: np.ndarray              # float32 [sum C, H_kv, d]
    v_chunk: np.ndarray
    # planted needles: rows (seq, kv_head, key position in seq history,
    # chunk token in seq it is aligned with)
    needles: np.ndarray = dataclasses.field(
        default_factory=lambda: np.zeros((0, 4), np.int64))

    @property
    def num_seqs(self) -> int:
        return int(self.cu_chunk.shape[0] - 1)

    @property
    def chunk_lens(self) -> List[int]:
        return [int(x) for x in np.diff(self.cu_chunk)]

    @property
    def hist_lens(self) -> List[int]:
        return [int(x) for x in np.diff(self.cu_hist)]


# name -> (seed offset, description); the generator recipe is in make_config
CONFIGS = {
    "tiny": 0,      # 1 seq, 1/1 heads, d=64, fp32, L=1024, C=128, Nq=16, B=128
    "llama8b": 1,   # 32/8 heads, d=128, bf16, L=32768, C=2048, Nq=64, B=2048
    "long": 2,      # 32/8 heads, d=128, bf16, L=131072, C=4096, Nq=128, B=4096
    "narrow": 3,    # 28/4 heads, d=128, bf16, L=65536, C=1024, Nq=32, B=1024
    "ragged": 4,    # 8 seqs, L={4..96}K, C=512 each, 32/8, Nq=32, B=1024
    "decode": 5,    # decode step (C=1): 8 seqs, 32/8 heads, d=128, bf16, L=16384, Nq=1, B=2048
}

SEED_BASE = 20260000


def _rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [T, H, d] at positions pos [T]."""
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]          # [T, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., :half].astype(np.float64)
    x2 = x[..., half:].astype(np.float64)
    out = np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)
    return out.astype(np.float32)


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_case(seqs: Sequence[Tuple[int, int]], num_q_heads: int,
              num_kv_heads: int, head_dim: int, dtype: str, n_q: int,
              budget: int, seed: int, *, scaled: bool = False,
              rope_base: Optional[float] = None, needles_per_head: int = 0,
              outlier_needles: float = 0.0, name: str = "case") -> Workload:
    """A workload of ragged sequences given as (chunk length, history length).

    Draw order (fixed, so a seed always gives the same arrays): channel
    scales, q, k_hist, v_hist, k_chunk, v_chunk, then the needles sequence by
    sequence and head by head.

    outlier_needles = a > 0 builds a crowd: per (sequence, KV head) a random
    unit direction u is drawn, a * u is added to every query head of the
    group and the needle tokens get -a * u instead, so the queries the needles
    align with point away from all the others.
    """
    if dtype not in ("fp32", "bf16"):
        raise ValueError(dtype)
    if num_q_heads % num_kv_heads:
        raise ValueError("H_q must be a multiple of H_kv")
    rng = np.random.Generator(np.random.PCG64(seed))
    H_q, H_kv, d = num_q_heads, num_kv_heads, head_dim
    G = H_q // H_kv
    C = [int(c) for c, _ in seqs]
    L = [int(l) for _, l in seqs]
    cu_chunk = np.concatenate([[0], np.cumsum(C)]).astype(np.int32)
    cu_hist = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
    TC, TL = int(cu_chunk[-1]), int(cu_hist[-1])

    sigma = None
    if scaled:
        sigma = np.exp(rng.uniform(math.log(0.5), math.log(4.0),
                                   size=(H_kv, d))).astype(np.float32)
    q = _normal(rng, (TC, H_q, d))
    k_hist = _normal(rng, (TL, H_kv, d))
    v_hist = _normal(rng, (TL, H_kv, d))
    k_chunk = _normal(rng, (TC, H_kv, d))
    v_chunk = _normal(rng, (TC, H_kv, d))
    if sigma is not None:
        q *= np.repeat(sigma, G, axis=0)[None, :, :]
        k_hist *= sigma[None, :, :]
        k_chunk *= sigma[None, :, :]
    if rope_base is not None:
        qpos = np.concatenate([np.arange(l, l + c) for c, l in zip(C, L)]) \
            if TC else np.zeros((0,), np.int64)
        hpos = np.concatenate([np.arange(0, l) for l in L]) \
            if TL else np.zeros((0,), np.int64)
        q = _rope(q, qpos, rope_base)
        k_chunk = _rope(k_chunk, qpos, rope_base)
        k_hist = _rope(k_hist, hpos, rope_base)

    planted = []
    if needles_per_head:
        for s in range(len(seqs)):
            if C[s] == 0 or L[s] == 0:
                continue
            n = min(needles_per_head, L[s])
            for h in range(H_kv):
                pos = rng.choice(L[s], size=n, replace=False)
                tok = rng.integers(0, C[s], size=n)
                noise = _normal(rng, (n, d))
                if outlier_needles > 0:
                    u = _normal(rng, (d,)).astype(np.float64)
                    u *= outlier_needles / np.linalg.norm(u)
                    sign = np.ones((C[s], 1, 1))
                    sign[tok] = -1.0
                    grp = q[cu_chunk[s]:cu_chunk[s + 1], h * G:(h + 1) * G, :]
                    grp += (sign * u[None, None, :]).astype(np.float32)
                if sigma is not None:
                    noise *= sigma[h][None, :]
                for i in range(n):
                    a = q[cu_chunk[s] + tok[i], h * G:(h + 1) * G, :] \
                        .astype(np.float64).sum(axis=0)
                    na = np.linalg.norm(a)
                    dirn = a / na if na > 0 else a
                    k_hist[cu_hist[s] + pos[i], h, :] = (
                        3.0 * math.sqrt(d) * dirn + noise[i]).astype(np.float32)
                    planted.append((s, h, int(pos[i]), int(tok[i])))

    if dtype == "bf16":
        q, k_hist, v_hist = round_to_bf16(q), round_to_bf16(k_hist), round_to_bf16(v_hist)
        k_chunk, v_chunk = round_to_bf16(k_chunk), round_to_bf16(v_chunk)
    return Workload(name=name, dtype=dtype, num_q_heads=H_q, num_kv_heads=H_kv,
                    head_dim=d, n_q=int(n_q), budget=int(budget),
                    cu_chunk=cu_chunk, cu_hist=cu_hist, q=q, k_hist=k_hist,
                    v_hist=v_hist, k_chunk=k_chunk, v_chunk=v_chunk,
                    needles=np.asarray(planted, np.int64).reshape(-1, 4))


def make_config(name: str) -> Workload:
    """One of the layer shapes, seeded with 20260000 + its index."""
    seed = SEED_BASE + CONFIGS[name]
    if name == "tiny":
        return _make_tiny(seed)
    if name == "llama8b":
        return make_case([(2048, 32768)], 32, 8, 128, "bf16", 64, 2048, seed,
                         scaled=True, name=name)
    if name == "long":
        return make_case([(4096, 131072)], 32, 8, 128, "bf16", 128, 4096, seed,
                         scaled=True, needles_per_head=64, name=name)
    if name == "narrow":
        return make_case([(1024, 65536)], 28, 4, 128, "bf16", 32, 1024, seed,
                         rope_base=1e6, name=name)
    if name == "ragged":
        hist = [k * 1024 for k in (4, 8, 16, 24, 32, 48, 64, 96)]
        return make_case([(512, l) for l in hist], 32, 8, 128, "bf16", 32, 1024,
                         seed, needles_per_head=16, name=name)
    if name == "decode":
        # the degenerate chunk of one token: its one (kept) query scores the
        # history; channel-scaled like llama8b
        return make_case([(1, 16384)] * 8, 32, 8, 128, "bf16", 1, 2048, seed,
                         scaled=True, name=name)
    raise KeyError(name)


def _make_tiny(seed: int) -> Workload:
    """1 seq, 1 query / 1 KV head, d=64, fp32, L=1024, C=128, Nq=16, B=128,
    with 8 needle keys, each aligned with its own randomly chosen chunk query:
    k = 3 * sqrt(d) * unit(q_c) + N(0, I)."""
    w = make_case([(128, 1024)], 1, 1, 64, "fp32", 16, 128, seed,
                  name="tiny")
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    pos = rng.choice(1024, size=8, replace=False)
    tok = rng.choice(128, size=8, replace=False)
    noise = _normal(rng, (8, 64))
    planted = []
    for i in range(8):
        a = w.q[tok[i], 0, :].astype(np.float64)
        w.k_hist[pos[i], 0, :] = (3.0 * 8.0 * a / np.linalg.norm(a)
                                  + noise[i]).astype(np.float32)
        planted.append((0, 0, int(pos[i]), int(tok[i])))
    w.needles = np.asarray(planted, np.int64)
    return w
