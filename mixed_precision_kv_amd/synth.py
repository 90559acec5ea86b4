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

Streams for one workload with seed ``s``: ``SeedSequence(s).spawn(4 + 4*steps)``
gives one child per array in the order keys, values, scores, queries, then
per append step (k_new, v_new, score_new, q_new).  An array is drawn in
chunks of 2**22 values (whole rows); chunk i uses ``PCG64(child.spawn(n)[i])``,
so the bytes do not depend on how many threads draw them.  fp32 normal draws
are cast to fp16 with round-to-nearest-even; the first ``outlier_channels``
key channels are multiplied by ``outlier_scale`` in fp32 before the cast.
Scores are fp32 ``exp(sigma * N(0,1))``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
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
    outlier_stride: int = 1           # outlier key channels at 0, stride, 2*stride, ...
    # channel rearrangement and clipped group ranges (tiered mode)
    reorder: bool = False             # store the channel orders of channel_orders()
    clip: float = 0.0                 # group min/max scale factor; 0: no clipping
    # pre-RoPE keys (tiered mode): rotary base; 0: keys used as given
    rope_theta: float = 0.0
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
W_SINGLE = BY_NAME["c1_single_head_t4096"]     # 1 x 4096 tokens, one KV head
W_LLAMA = BY_NAME["c2_llama8b_b8_t32k"]        # 8 x 32768 tokens, Llama-3.1-8B-shaped layer
W_LONG = BY_NAME["c3_long_b1_t128k"]           # 1 x 131072 tokens, 8/6 levels, G 64
W_APPEND = BY_NAME["c4_append_b64_t16k"]       # 64 x 16384 prefix + 256 appends
W_KCHAN = BY_NAME["c5_kchan_b4_t64k"]          # 4 x 65536, per-channel keys
# The Llama-shaped layer with rearranged channels and clipped group ranges
# (SKVQ abstract): one outlier key channel in every group of 32 in the input,
# brought into one group by the stored order; clip factor 0.9.
W_SKVQ = W_LLAMA.shrink(name="skvq_llama8b_b8_t32k", outlier_stride=32, reorder=True, clip=0.9)
BY_NAME[W_SKVQ.name] = W_SKVQ
# The Llama-shaped layer and the long-context workload with pre-RoPE keys
# (KVQuant summary, "techniques"): keys drawn as above stand for the keys
# before the rotary embedding; Llama-3.1's rotary base 500000.
W_ROPE = W_LLAMA.shrink(name="rope_llama8b_b8_t32k", rope_theta=500000.0)
W_ROPE_LONG = W_LONG.shrink(name="rope_long_b1_t128k", rope_theta=500000.0)
BY_NAME[W_ROPE.name] = W_ROPE
BY_NAME[W_ROPE_LONG.name] = W_ROPE_LONG


CHUNK = 1 << 22
_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _draw_f16(seq: np.random.SeedSequence, shape, col_scale=None) -> np.ndarray:
    """N(0,1) fp32 draws (optionally scaled per last-axis channel in fp32)
    cast to fp16 (RNE), chunk by chunk from independent child streams."""
    out = np.empty(shape, dtype=np.float16)
    flat = out.reshape(-1)
    n = flat.size
    nchunk = max(1, -(-n // CHUNK))
    kids = seq.spawn(nchunk)
    D = shape[-1]
    assert CHUNK % D == 0

    def job(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        x = np.random.Generator(np.random.PCG64(kids[i])).standard_normal(hi - lo, dtype=np.float32)
        if col_scale is not None:
            x = (x.reshape(-1, D) * col_scale).reshape(-1)
        flat[lo:hi] = x.astype(np.float16)

    if nchunk == 1:
        job(0)
    else:
        with ThreadPoolExecutor(_WORKERS) as ex:
            list(ex.map(job, range(nchunk)))
    return out


def _draw_scores(seq: np.random.SeedSequence, shape, sigma: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seq))
    return np.exp(np.float32(sigma) * g.standard_normal(shape, dtype=np.float32)).astype(np.float32)


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
    B, T, H, Hq, D = w.batch, w.tokens, w.kv_heads, w.q_heads, w.head_dim
    n_steps = w.append_steps if steps is None else min(steps, w.append_steps)
    kids = np.random.SeedSequence(w.seed).spawn(4 + 4 * w.append_steps)
    col = np.ones(D, dtype=np.float32)
    col[:w.outlier_channels * w.outlier_stride:w.outlier_stride] = np.float32(w.outlier_scale)
    k = _draw_f16(kids[0], (B, T, H, D), col)
    v = _draw_f16(kids[1], (B, T, H, D))
    scores = _draw_scores(kids[2], (B, T), w.score_sigma) if w.mode == TIERED else None
    q = _draw_f16(kids[3], (B, Hq, D))
    st = []
    for i in range(n_steps):
        c = kids[4 + 4 * i: 8 + 4 * i]
        st.append(dict(k_new=_draw_f16(c[0], (B, H, D)), v_new=_draw_f16(c[1], (B, H, D)),
                       score_new=_draw_scores(c[2], (B,), 1.0), q=_draw_f16(c[3], (B, Hq, D))))
    return Inputs(k=k, v=v, scores=scores, q=q, steps=st)


def make_queries(w: Workload, n_queries: int, seed: int = 1) -> np.ndarray:
    """A block of new query tokens per sequence, fp16 N(0,1) [B][M][Hq][D]
    (the next turn's tokens reading the cache); a stream of its own, so the
    cache inputs of the workload are unchanged."""
    ss = np.random.SeedSequence([w.seed, 1000 + seed])
    return _draw_f16(ss, (w.batch, n_queries, w.q_heads, w.head_dim))


def channel_orders(w: Workload) -> np.ndarray:
    """Stored channel orders int32 [2][Hkv][D] (keys, values) standing in for
    an order calibrated offline: keys put the input's outlier channels first
    (ascending), then the others ascending; values take a seeded random order
    per KV head (their channels are alike, so it only exercises the layout).
    Entry p is the input channel stored at position p."""
    D, H = w.head_dim, w.kv_heads
    out = np.empty((2, H, D), dtype=np.int32)
    outl = np.arange(w.outlier_channels) * w.outlier_stride
    rest = np.setdiff1d(np.arange(D), outl)
    out[0] = np.concatenate([outl, rest])[None, :]
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 2000])))
    for h in range(H):
        out[1, h] = g.permutation(D)
    return out
