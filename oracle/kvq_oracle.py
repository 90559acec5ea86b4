"""CPU oracle for semantic mixed-precision KV-cache quantization and decode
attention over the packed cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library.

Plain, slow, obviously-correct numpy.  Every function states the passage it
follows.  Sources (cited by page title and section):

* [SemKV] "SemKV: Semantic Mixed-Precision KV Cache Quantization Guided by
  the Quality Cliff for Long-Context LLM Inference" (arXiv 2608.28911),
  Abstract: uniform affine quantization on a fractional-bit grid measured in
  "code bits/value" (2.322 and 2.0 are the two grids around the cliff);
  every token is preserved; tokens are ranked by a model-internal score and
  given one of two adjacent above-cliff precisions; quantization also happens
  at generation time.
* [SKVQ] "SKVQ: Sliding-window Key and Value Cache Quantization for Large
  Language Models" (arXiv 2405.06219), Abstract: the most recent window of
  tokens is kept in high precision; 2-bit keys and 1.5-bit values.
* [KVQuant] KVQuant summary (lianzai.com post), "techniques" paragraph:
  per-channel key quantization; per-vector dense-and-sparse quantization
  with a per-vector outlier threshold, outliers stored sparsely.

Readings of what the pages leave open (each is the plainest one the rest
supports; all are listed in the design notes):

* L-level grid: code bits = log2(L); codes 0..L-1.
* Affine group quantizer: zero z = group minimum (fp16), scale
  s = fp16_rne(fp32(max - min) / fp32(L - 1)); code
  c = clamp(rint_even(fp32(x - z) / fp32(s)), 0, L - 1); s == 0 -> all codes 0.
  Dequantized value x^ = z + c*s (exact in fp64).  Min/max use the IEEE total
  order (-0 < +0).
* Base-L packing: a word holds n_L = max{n : L^n <= 2^32} codes, little-endian
  digits (code j has weight L^j), unused digits 0.  Keys are packed along the
  head dimension of one token (row words); values are packed along the slot
  axis of one channel (column words).
* Rank: stable descending order of the fp32 score; equal scores keep token
  order.  Top tier <=> rank < n_hi.  Slot = index within the tier in token
  order.  Token map entry = slot | tier << 31 (tier 0 = hi, 1 = lo).
* Running median (generation time): median of the scores already in the
  sequence; even count -> mean of the two middle values in fp64; the new token
  takes the high grid iff its score is strictly greater.
* kchan mode: n_q = k_block * floor((T - window) / k_block) tokens quantized,
  the rest kept fp16; per key vector the ``sparse_per_vec`` entries of largest
  |x| (ties -> lower channel) are stored as (channel, fp16) and zeroed in the
  dense part; dense keys are quantized per (channel, k_block-token block);
  values per token in groups of v_group.  k^ = deq(dense) + sparse.
* Attention: o = softmax(scale * q . k^) v^ in fp64 over every cached token,
  query head hq reads KV head hq // (Hq / Hkv).
* [KVQuant] "techniques", pre-RoPE keys (tiered mode, optional): keys are
  stored as given (before the rotary embedding) and rotated at attention time
  by their token positions (adjacent channel pairs, theta_i = base^(-2i/D));
  the query is given already rotated.
* [SKVQ] Abstract, channel rearrangement and clipped group ranges (tiered
  mode, optional): a fixed channel order per KV head for keys and for values
  (stored position p holds channel order[p]; groups are runs of G positions);
  the group minimum and maximum are each scaled by a clip factor in (0, 1]
  (fp32 product, fp16 RNE) before the grid is formed, values outside take the
  end codes.
"""
from __future__ import annotations

import bisect
import math

import numpy as np

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------- grids -----
def code_bits(L: int) -> float:
    """[SemKV] Abstract: precision of an L-level grid in code bits per value."""
    return math.log2(L)


def codes_per_word(L: int) -> int:
    """Largest n with L**n <= 2**32 (base-L digits that fit one 32-bit word)."""
    n = 0
    while L ** (n + 1) <= 2 ** 32:
        n += 1
    return n


def words_per_row(L: int, D: int) -> int:
    """Words holding one D-value row, packed along the row."""
    n = codes_per_word(L)
    return -(-D // n)


# ------------------------------------------------------------ quantizer -----
def _f16_total_order_key(x16: np.ndarray) -> np.ndarray:
    """Integer key whose order is the IEEE total order of finite fp16 values
    (-0 sorts below +0)."""
    b = x16.view(np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF) - 1, b)


def quantize_groups(x16: np.ndarray, L: int, clip=None):
    """[SemKV] Abstract (uniform affine quantizer on an L-level grid), applied
    to every group along the last axis.

    clip (0 < clip <= 1, or None): [SKVQ] Abstract, clipped dynamic
    quantization at the group level.  Reading: the group's minimum and maximum
    are each multiplied by clip in fp32 and rounded to fp16 (RNE) before the
    grid is formed from them; values outside the clipped range take the end
    codes 0 and L - 1.  clip = 1 leaves both unchanged.

    x16: fp16 [..., G].  Returns (codes uint8 [..., G], scale fp16 [...],
    zero fp16 [...]).
    """
    assert x16.dtype == np.float16
    assert np.all(np.isfinite(x16)), "inputs must be finite"
    key = _f16_total_order_key(x16)
    i_mn = np.argmin(key, axis=-1)[..., None]
    i_mx = np.argmax(key, axis=-1)[..., None]
    mn = np.take_along_axis(x16, i_mn, axis=-1)[..., 0]
    mx = np.take_along_axis(x16, i_mx, axis=-1)[..., 0]
    if clip is not None:
        assert 0.0 < clip <= 1.0
        mn = (mn.astype(F32) * F32(clip)).astype(np.float16)   # fp32 product, then fp16 RNE
        mx = (mx.astype(F32) * F32(clip)).astype(np.float16)
    rng32 = mx.astype(F32) - mn.astype(F32)            # fp32, round to nearest even
    s32 = rng32 / F32(L - 1)                            # IEEE fp32 division
    s16 = s32.astype(np.float16)                        # RNE, subnormals kept
    assert np.all(np.isfinite(s16)), "group scale overflows fp16"
    z16 = mn
    a = x16.astype(F32) - z16.astype(F32)[..., None]    # fp32
    sf = s16.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = a / sf                                      # IEEE fp32 division
    c = np.rint(q)                                      # ties to even
    c = np.clip(c, 0, L - 1)
    c = np.where(sf == 0, 0, c)
    return c.astype(np.uint8), s16, z16


def dequantize_groups(codes: np.ndarray, scale16: np.ndarray, zero16: np.ndarray) -> np.ndarray:
    """x^ = z + c * s, evaluated exactly in fp64."""
    return zero16.astype(F64)[..., None] + codes.astype(F64) * scale16.astype(F64)[..., None]


# --------------------------------------------------------------- packing ----
def pack_digits(codes: np.ndarray, L: int) -> np.ndarray:
    """One base-L word from the last axis (length <= n_L): sum_j c_j * L**j."""
    n = codes.shape[-1]
    assert n <= codes_per_word(L)
    w = np.zeros(codes.shape[:-1], dtype=np.uint64)
    for j in range(n - 1, -1, -1):                     # Horner, most significant first
        w = w * np.uint64(L) + codes[..., j].astype(np.uint64)
    assert np.all(w < np.uint64(2 ** 32))
    return w.astype(np.uint32)


def unpack_digits(words: np.ndarray, L: int, n: int) -> np.ndarray:
    w = words.astype(np.uint64)
    out = np.empty(words.shape + (n,), dtype=np.uint8)
    for j in range(n):
        out[..., j] = (w % np.uint64(L)).astype(np.uint8)
        w //= np.uint64(L)
    return out


def pack_rows(codes: np.ndarray, L: int) -> np.ndarray:
    """Row words: codes [N][D] -> [N][ceil(D/n_L)], packed along D."""
    N, D = codes.shape
    n = codes_per_word(L)
    W = -(-D // n)
    padded = np.zeros((N, W * n), dtype=np.uint8)
    padded[:, :D] = codes
    return pack_digits(padded.reshape(N, W, n), L)


def pack_cols(codes: np.ndarray, L: int) -> np.ndarray:
    """Column words: codes [N][D] -> [ceil(N/n_L)][D], packed along the slot axis."""
    N, D = codes.shape
    n = codes_per_word(L)
    R = -(-N // n)
    padded = np.zeros((R * n, D), dtype=np.uint8)
    padded[:N] = codes
    return pack_digits(padded.reshape(R, n, D).transpose(0, 2, 1), L)


# ------------------------------------------------------------------ rank ----
def rank_desc(scores: np.ndarray) -> np.ndarray:
    """[SemKV] Abstract ("ranks tokens by a model-internal score"): position of
    each token in descending score order, equal scores in token order.
    scores fp32 [B][T] -> int32 [B][T]."""
    B, T = scores.shape
    order = np.argsort(-scores, axis=1, kind="stable")
    rank = np.empty((B, T), dtype=np.int32)
    np.put_along_axis(rank, order, np.arange(T, dtype=np.int32)[None, :].repeat(B, 0), axis=1)
    return rank


def tiers_and_slots(rank: np.ndarray, n_hi: int):
    """[SemKV] Abstract ("preserves every token ... assigns two adjacent
    precisions"): tier 0 (high grid) iff rank < n_hi, else tier 1; slot is the
    index among same-tier tokens in token order.

    Returns tokmap uint32 [B][T] (slot | tier<<31), counts int32 [B][2],
    and inv: list over b of (tokens_hi, tokens_lo) int arrays (slot -> token).
    """
    B, T = rank.shape
    tokmap = np.empty((B, T), dtype=np.uint32)
    counts = np.empty((B, 2), dtype=np.int32)
    inv = []
    for b in range(B):
        lo = rank[b] >= n_hi
        t_hi = np.nonzero(~lo)[0]
        t_lo = np.nonzero(lo)[0]
        tokmap[b, t_hi] = np.arange(len(t_hi), dtype=np.uint32)
        tokmap[b, t_lo] = np.arange(len(t_lo), dtype=np.uint32) | np.uint32(1 << 31)
        counts[b] = (len(t_hi), len(t_lo))
        inv.append((t_hi, t_lo))
    return tokmap, counts, inv


# ------------------------------------------------------ tiered cache unit ---
class Pool:
    """Canonical contents of one tier pool of one (sequence, KV head).

    order_k / order_v (int [D] or None): [SKVQ] Abstract, the channels of
    the KV cache rearranged so that the channels sharing a quantization group
    are alike.  Reading: a fixed order per KV head for keys and one for values;
    position p of a stored row holds channel order[p], so groups are runs of G
    positions in that order and the codes are stored in it.  ``k_hat`` and
    ``v_hat`` return rows in the original channel order.  clip: see
    ``quantize_groups``."""

    def __init__(self, L: int, G: int, D: int, order_k=None, order_v=None, clip=None):
        self.L, self.G, self.D = L, G, D
        self.order_k = None if order_k is None else np.asarray(order_k, dtype=np.int64)
        self.order_v = None if order_v is None else np.asarray(order_v, dtype=np.int64)
        for o in (self.order_k, self.order_v):
            assert o is None or np.array_equal(np.sort(o), np.arange(D)), "not a permutation"
        self.clip = clip
        self.k_codes = np.zeros((0, D), np.uint8)
        self.k_scale = np.zeros((0, D // G), np.float16)
        self.k_zero = np.zeros((0, D // G), np.float16)
        self.v_codes = np.zeros((0, D), np.uint8)
        self.v_scale = np.zeros((0, D // G), np.float16)
        self.v_zero = np.zeros((0, D // G), np.float16)

    @property
    def n(self) -> int:
        return self.k_codes.shape[0]

    def add_rows(self, k16: np.ndarray, v16: np.ndarray):
        """Quantize rows [N][D] (per-token groups of G) and append them."""
        N = k16.shape[0]
        if N == 0:
            return
        ng = self.D // self.G
        if self.order_k is not None:
            k16 = k16[:, self.order_k]                  # stored position p <- channel order[p]
        if self.order_v is not None:
            v16 = v16[:, self.order_v]
        kc, ks, kz = quantize_groups(k16.reshape(N, ng, self.G), self.L, self.clip)
        vc, vs, vz = quantize_groups(v16.reshape(N, ng, self.G), self.L, self.clip)
        self.k_codes = np.concatenate([self.k_codes, kc.reshape(N, self.D)])
        self.k_scale = np.concatenate([self.k_scale, ks])
        self.k_zero = np.concatenate([self.k_zero, kz])
        self.v_codes = np.concatenate([self.v_codes, vc.reshape(N, self.D)])
        self.v_scale = np.concatenate([self.v_scale, vs])
        self.v_zero = np.concatenate([self.v_zero, vz])

    def k_words(self):
        return pack_rows(self.k_codes, self.L)

    def v_words(self):
        return pack_cols(self.v_codes, self.L)

    @staticmethod
    def _original_order(rows, order):
        if order is None:
            return rows
        out = np.empty_like(rows)
        out[:, order] = rows                            # channel order[p] <- stored position p
        return out

    def k_hat(self):
        N, ng = self.n, self.D // self.G
        deq = dequantize_groups(self.k_codes.reshape(N, ng, self.G), self.k_scale,
                                self.k_zero).reshape(N, self.D)
        return self._original_order(deq, self.order_k)

    def v_hat(self):
        N, ng = self.n, self.D // self.G
        deq = dequantize_groups(self.v_codes.reshape(N, ng, self.G), self.v_scale,
                                self.v_zero).reshape(N, self.D)
        return self._original_order(deq, self.order_v)


def quantize_tiered_unit(k_unit: np.ndarray, v_unit: np.ndarray, inv_b, L_hi: int, L_lo: int,
                         G: int, order_k=None, order_v=None, clip=None):
    """[SemKV] Abstract: every token of one (sequence, KV head) is quantized on
    its tier's grid and stored, none dropped.  k_unit, v_unit fp16 [T][D];
    inv_b = (tokens_hi, tokens_lo) in slot order.  Channel orders and clip as
    in ``Pool`` (None: the plain quantizer).  Returns (Pool hi, Pool lo)."""
    D = k_unit.shape[1]
    pools = (Pool(L_hi, G, D, order_k, order_v, clip), Pool(L_lo, G, D, order_k, order_v, clip))
    for p, toks in enumerate(inv_b):
        pools[p].add_rows(k_unit[toks], v_unit[toks])
    return pools


# ------------------------------------------------------------- attention ----
def attention_fp64(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float) -> np.ndarray:
    """Plain softmax attention of a group of query heads over one KV head, fp64.
    q [Hg][D], k_hat/v_hat [N][D] -> [Hg][D]."""
    s = (q.astype(F64) @ k_hat.astype(F64).T) * F64(scale)   # [Hg][N]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ v_hat.astype(F64)) / p.sum(axis=1, keepdims=True)


def decode_unit(q_group: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float):
    """Decode attention for the Hq/Hkv query heads that read one KV head."""
    return attention_fp64(q_group, k_hat, v_hat, scale)


def attention_lse_fp64(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float):
    """Attention of a block of query rows over the whole cache, with each
    row's log-sum-exp, fp64: the cached history of one KV head read by several
    new query tokens at once (a multi-turn continuation re-reading the cache,
    [SemKV] Abstract).  Rows are independent; no mask, since every cached
    token precedes the new ones.  q [R][D] -> (o [R][D], lse [R]) with
    lse = ln sum_t exp(scale q . k^_t), so that a caller can merge o with
    attention over the new tokens themselves."""
    s = (q.astype(F64) @ k_hat.astype(F64).T) * F64(scale)   # [R][N]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v_hat.astype(F64)) / l, (m + np.log(l))[:, 0]


def token_attention_mass(q_seq: np.ndarray, k_hat_heads, scale: float) -> np.ndarray:
    """Per-token importance from one decode step: the attention weight each
    cached token receives, summed over every query head of the sequence, fp64
    ([SemKV] Abstract: tokens are ranked by a model-internal score; this is
    the score decode itself can report).  q_seq [Hq][D]; k_hat_heads: list of
    Hkv arrays [N][D] in token order; query head hq reads KV head
    hq // (Hq / Hkv).  Returns [N]; it sums to Hq."""
    Hq = q_seq.shape[0]
    g = Hq // len(k_hat_heads)
    mass = np.zeros(k_hat_heads[0].shape[0], dtype=F64)
    for hq in range(Hq):
        s = (k_hat_heads[hq // g].astype(F64) @ q_seq[hq].astype(F64)) * F64(scale)
        p = np.exp(s - s.max())
        mass += p / p.sum()
    return mass


# -------------------------------------------------- pre-RoPE keys (KVQuant) ---
def rope_thetas(D: int, base: float) -> np.ndarray:
    """Rotary frequencies of the D/2 channel pairs, fp64: theta_i =
    base ** (-2 i / D).  [KVQuant] summary, "techniques" (Pre-RoPE Key
    Quantization: keys are quantized before the rotary position embedding,
    which mixes channels).  The pages give no formula; this is the standard
    rotary embedding (pairs of adjacent channels (2i, 2i + 1), each turned by
    the angle position * theta_i)."""
    i = np.arange(D // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / F64(D))


def rope_rotate(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rows x [N][D] (fp64) turned by their positions [N]: pair i of row t,
    (x[2i], x[2i+1]), becomes (x cos a - y sin a, x sin a + y cos a) with
    a = positions[t] * theta_i.  Position 0 is the identity."""
    x = np.asarray(x, dtype=F64)
    N, D = x.shape
    ang = np.asarray(positions, dtype=F64)[:, None] * rope_thetas(D, base)[None, :]   # [N][D/2]
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = xe * c - xo * s
    out[:, 1::2] = xe * s + xo * c
    return out


def row_rel_err(o: np.ndarray, r: np.ndarray) -> float:
    """Error measure for attention outputs: max over rows of
    max|o - r| / max|r| (rows are the last-but-one axis)."""
    o = o.astype(F64).reshape(-1, o.shape[-1])
    r = r.astype(F64).reshape(-1, r.shape[-1])
    den = np.abs(r).max(axis=1)
    num = np.abs(o - r).max(axis=1)
    return float((num / np.where(den == 0, 1.0, den)).max())


# --------------------------------------------- generation-time append -------
class RunningMedian:
    """Sorted scores of one sequence ([SemKV] Abstract: quantization at
    generation time).  The new token's tier is decided against the median of
    the scores already present (mean of the two middle ones for an even
    count, in fp64); strictly greater -> high grid."""

    def __init__(self, scores_f32):
        self.s = sorted(float(x) for x in np.asarray(scores_f32, dtype=F32))

    def median(self) -> float:
        n = len(self.s)
        a, b = self.s[(n - 1) // 2], self.s[n // 2]
        return (a + b) * 0.5

    def decide_and_insert(self, s_new: float) -> int:
        """Returns tier (0 = hi, 1 = lo) and records the score."""
        s_new = float(F32(s_new))
        tier = 0 if s_new > self.median() else 1
        bisect.insort(self.s, s_new)
        return tier


# ------------------------------------------------------------ kchan mode ----
def kchan_quantized_count(T: int, window: int, k_block: int) -> int:
    """[SKVQ] Abstract (recent window kept in high precision): whole k_block
    token blocks before the fp16 window are quantized."""
    return k_block * max(0, (T - window) // k_block)


def split_sparse(k16: np.ndarray, per_vec: int):
    """[KVQuant] per-vector dense-and-sparse: in each key vector (row) the
    ``per_vec`` entries of largest magnitude (ties -> lower channel) are kept
    exactly; the dense part has +0 there.  Returns (dense fp16 [N][D],
    channels int [N][per_vec] ascending, values fp16 [N][per_vec])."""
    N, D = k16.shape
    mag = (k16.view(np.uint16) & 0x7FFF).astype(np.int32)
    # stable sort by descending magnitude keeps lower channels first among ties
    order = np.argsort(-mag, axis=1, kind="stable")[:, :per_vec]
    ch = np.sort(order, axis=1)
    vals = np.take_along_axis(k16, ch, axis=1)
    dense = k16.copy()
    np.put_along_axis(dense, ch, np.float16(0.0), axis=1)
    return dense, ch, vals


class KChanUnit:
    """Canonical kchan-mode contents of one (sequence, KV head)."""

    def __init__(self, k_unit, v_unit, w):
        T, D = k_unit.shape
        self.D = D
        self.n_q = nq = kchan_quantized_count(T, w.window, w.k_block)
        self.k_levels, self.v_levels = w.k_levels, w.v_levels
        self.k_block, self.v_group = w.k_block, w.v_group
        dense, self.sp_ch, self.sp_val = split_sparse(k_unit[:nq], w.sparse_per_vec)
        nb = nq // w.k_block
        # [KVQuant] per-channel key quantization: groups run along tokens
        blk = dense.reshape(nb, w.k_block, D).transpose(0, 2, 1)        # [nb][D][k_block]
        kc, self.k_scale, self.k_zero = quantize_groups(np.ascontiguousarray(blk), w.k_levels)
        self.k_codes = kc.transpose(0, 2, 1).reshape(nq, D)               # [n_q][D]
        vc, self.v_scale, self.v_zero = quantize_groups(
            v_unit[:nq].reshape(nq, D // w.v_group, w.v_group), w.v_levels) if nq else (
            np.zeros((0, D // w.v_group, w.v_group), np.uint8), np.zeros((0, D // w.v_group), np.float16),
            np.zeros((0, D // w.v_group), np.float16))
        self.v_codes = vc.reshape(nq, D)
        self.k_win = k_unit[nq:].copy()
        self.v_win = v_unit[nq:].copy()

    def k_words(self):
        return pack_rows(self.k_codes, self.k_levels)

    def v_words(self):
        return pack_cols(self.v_codes, self.v_levels)

    def k_hat(self):
        nq, D = self.k_codes.shape
        nb = nq // self.k_block
        c = self.k_codes.reshape(nb, self.k_block, D).transpose(0, 2, 1)
        deq = dequantize_groups(c, self.k_scale, self.k_zero).transpose(0, 2, 1).reshape(nq, D)
        np.put_along_axis(deq, self.sp_ch,
                          np.take_along_axis(deq, self.sp_ch, axis=1) + self.sp_val.astype(F64), axis=1)
        return np.concatenate([deq, self.k_win.astype(F64)])

    def v_hat(self):
        nq, D = self.v_codes.shape
        deq = dequantize_groups(self.v_codes.reshape(nq, D // self.v_group, self.v_group), self.v_scale,
                                self.v_zero).reshape(nq, D)
        return np.concatenate([deq, self.v_win.astype(F64)])


# -------------------------------------------------------------- storage -----
def tiered_unit_bytes(n_hi: int, n_lo: int, L_hi: int, L_lo: int, G: int, D: int) -> int:
    """Bytes one (sequence, KV head) occupies: row key words, column value
    words, and one fp16 (scale, zero) pair per group for keys and values."""
    total = 0
    for n, L in ((n_hi, L_hi), (n_lo, L_lo)):
        total += n * words_per_row(L, D) * 4                 # key words
        total += -(-n // codes_per_word(L)) * D * 4          # value words
        total += 2 * n * (D // G) * 4                        # K and V (scale, zero)
    return total


def kchan_unit_bytes(T: int, w, D: int) -> int:
    nq = kchan_quantized_count(T, w.window, w.k_block)
    b = nq * words_per_row(w.k_levels, D) * 4                 # key words
    b += (nq // w.k_block) * D * 4                            # per-channel (scale, zero)
    b += nq * w.sparse_per_vec * 4                            # (channel, fp16) entries
    b += -(-nq // codes_per_word(w.v_levels)) * D * 4         # value words
    b += nq * (D // w.v_group) * 4                            # value (scale, zero)
    b += (T - nq) * D * 2 * 2                                 # fp16 window, K and V
    return b


def storage_ratio(fp16_bytes: int, packed_bytes: int) -> float:
    return fp16_bytes / packed_bytes
