"""Seeded synthetic inputs for the mixed-precision KV-cache path.

This module only draws random numbers and casts them to the storage types
(fp16 keys/values/queries, fp32 scores).  It holds none of the method's
arithmetic: no ranking, no quantizer, no packing, no attention.  Both the
CPU oracle (``oracle/``) and the HIP path consume exactly the bytes produced
here.

Workloads (one per entry of ``CONFIGS``) follow the SemKV setting (SemKV
abstract: Llama-3.1-8B-Instruct-shaped KV cache, per-token model-internal
scores, two adjacent fractional-bit grids) and, for ``kchan``, the KVQuant
per-channel-key / dense-and-sparse scheme (KVQuant summary, "techniques")
with the SKVQ high-precision recent window (SKVQ abstract).

Draw order for one workload with seed ``s`` (numpy ``Generator(PCG64(s))``):
keys, values, scores, queries, then per append step (k_new, v_new, score_new,
q_new).  fp32 normal draws are cast to fp16 with round-to-nearest-even; the
first ``outlier_channels`` key channels are multiplied by ``outlier_scale``
in fp32 before the cast.  Scores are fp32 ``exp(sigma * N(0,1))``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

TIERED = "tiered"
KCHAN = "kchan"


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    kv_heads: int
    q_heads: int
    head_dim: int
    tokens: int                       # context length T before any append
    mode: str = TIERED
    # tiered mode: two adjacent grids, per-token groups along head_dim
    levels_hi: int = 6
    levels_lo: int = 5
    group: int = 32
    frac_hi: float = 0.5              # n_hi = floor(frac_hi * T)
    score_sigma: float = 1.0
    # generation-time append (tiered mode)
    append_steps: int = 0
    # kchan mode (per-channel keys, dense-and-sparse, fp16 window)
    k_levels: int = 4
    k_block: int = 128
    v_levels: int = 3
    v_group: int = 32
    window: int = 128
    sparse_per_vec: int = 2           # ceil(1% of head_dim=128)
    # input distribution
    outlier_channels: int = 4
    outlier_scale: float = 10.0
    seed: int = 0

    @property
    def n_hi(self) -> int:
        return int(np.floor(self.frac_hi * self.tokens))

    @property
    def capacity(self) -> int:
        return self.tokens + self.append_steps

    def shrink(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  Index 1 (Llama-3.1-8B-shaped decode layer) is the one
# the headline throughput is quoted on.
CONFIGS = [
    Workload("c1_single_head_t4096", batch=1, kv_heads=1, q_heads=4, head_dim=128,
             tokens=4096, levels_hi=6, levels_lo=5, group=32, frac_hi=0.5),
    Workload("c2_llama8b_b8_t32k", batch=8, kv_heads=8, q_heads=32, head_dim=128,
             tokens=32768, levels_hi=6, levels_lo=5, group=32, frac_hi=0.5),
    Workload("c3_long_b1_t128k", batch=1, kv_heads=8, q_heads=32, head_dim=128,
             tokens=131072, levels_hi=8, levels_lo=6, group=64, frac_hi=0.25,
             score_sigma=2.0),
    Workload("c4_append_b64_t16k", batch=64, kv_heads=8, q_heads=32, head_dim=128,
             tokens=16384, levels_hi=6, levels_lo=5, group=32, frac_hi=0.5,
             append_steps=256),
    Workload("c5_kchan_b4_t64k", batch=4, kv_heads=8, q_heads=32, head_dim=128,
             tokens=65536, mode=KCHAN, k_levels=4, k_block=128, v_levels=3,
             v_group=32, window=128, sparse_per_vec=2),
]
BY_NAME = {w.name: w for w in CONFIGS}


def _f16_normal(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) fp32 draws cast to fp16 (RNE), generated in chunks to bound memory."""
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1)
    for i in range(0, flat.size, chunk):
        n = min(chunk, flat.size - i)
        flat[i:i + n] = rng.standard_normal(n, dtype=np.float32).astype(np.float16)
    return out


def _f16_normal_outliers(rng, shape, n_out: int, scale: float, chunk_rows: int = 1 << 17):
    """Like ``_f16_normal`` but the first ``n_out`` channels (last axis) are
    multiplied by ``scale`` in fp32 before the fp16 cast."""
    out = np.empty(shape, dtype=np.float16)
    D = shape[-1]
    rows = out.reshape(-1, D)
    sc = np.ones(D, dtype=np.float32)
    sc[:n_out] = np.float32(scale)
    for i in range(0, rows.shape[0], chunk_rows):
        n = min(chunk_rows, rows.shape[0] - i)
        x = rng.standard_normal((n, D), dtype=np.float32)
        x *= sc
        rows[i:i + n] = x.astype(np.float16)
    return out


@dataclass
class Inputs:
    """Host arrays for one workload.

    k, v:    fp16 [B][T][Hkv][D] (token-major, as a prefill produces them)
    scores:  fp32 [B][T]  (None in kchan mode)
    q:       fp16 [B][Hq][D]
    steps:   list of per-append-step dicts with k_new/v_new fp16 [B][Hkv][D],
             score_new fp32 [B], q fp16 [B][Hq][D]
    """
    k: np.ndarray
    v: np.ndarray
    scores: Optional[np.ndarray]
    q: np.ndarray
    steps: list = field(default_factory=list)


def make_inputs(w: Workload, steps: Optional[int] = None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, T, H, Hq, D = w.batch, w.tokens, w.kv_heads, w.q_heads, w.head_dim
    k = _f16_normal_outliers(rng, (B, T, H, D), w.outlier_channels, w.outlier_scale)
    v = _f16_normal(rng, (B, T, H, D))
    scores = None
    if w.mode == TIERED:
        scores = np.exp(np.float32(w.score_sigma) *
                        rng.standard_normal((B, T), dtype=np.float32)).astype(np.float32)
    q = _f16_normal(rng, (B, Hq, D))
    n_steps = w.append_steps if steps is None else min(steps, w.append_steps)
    st = []
    for _ in range(n_steps):
        kn = _f16_normal(rng, (B, H, D))
        vn = _f16_normal(rng, (B, H, D))
        sn = np.exp(rng.standard_normal(B, dtype=np.float32)).astype(np.float32)
        qn = _f16_normal(rng, (B, Hq, D))
        st.append(dict(k_new=kn, v_new=vn, score_new=sn, q=qn))
    return Inputs(k=k, v=v, scores=scores, q=q, steps=st)
