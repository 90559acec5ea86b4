"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (values the pages print, closed forms, exact-rational
arithmetic, brute force, library routines, invariants)."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import kvq_oracle as O
from mixed_precision_kv_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------- grids ---
def test_code_bits_match_printed_values():
    for L, printed, decimals in _golden("code_bits.txt"):
        assert round(O.code_bits(int(L)), int(decimals)) == float(printed)


def test_codes_per_word_table():
    for L, n, W in _golden("codes_per_word.txt"):
        L, n, W = int(L), int(n), int(W)
        assert O.codes_per_word(L) == n
        assert O.words_per_row(L, 128) == W
    for L in range(3, 17):
        n = O.codes_per_word(L)
        assert L ** n <= 2 ** 32 < L ** (n + 1)


# --------------------------------------------------------------- packing ---
@pytest.mark.parametrize("L", [3, 4, 5, 6, 8])
def test_pack_exhaustive_small(L):
    """Every code triple: the word equals Python's own base-L parse of the
    digit string (most significant digit first), and unpacks back."""
    codes = np.array(list(itertools.product(range(L), repeat=3)), dtype=np.uint8)
    w = O.pack_digits(codes, L)
    ref = [int("".join(str(d) for d in row[::-1]), L) for row in codes]
    assert w.tolist() == ref
    assert np.array_equal(O.unpack_digits(w, L, 3), codes)


@pytest.mark.parametrize("L", [3, 4, 5, 6, 8])
def test_pack_full_word_and_rows(L):
    rng = np.random.default_rng(L)
    n = O.codes_per_word(L)
    codes = rng.integers(0, L, size=(500, n), dtype=np.uint8)
    codes[0] = L - 1                                 # largest word L^n - 1
    w = O.pack_digits(codes, L)
    assert int(w[0]) == L ** n - 1
    ref = [sum(int(c) * L ** j for j, c in enumerate(row)) for row in codes]
    assert w.tolist() == ref
    # rows pack along D, columns along the slot axis: transposes of each other
    c2 = rng.integers(0, L, size=(2 * n + 3, 2 * n + 3), dtype=np.uint8)
    assert np.array_equal(O.pack_rows(c2, L), O.pack_cols(c2.T.copy(), L).T)
    # padding digits are zero: the last row word only holds the tail codes
    row = O.pack_rows(c2[:1], L)[0]
    tail = c2[0, (len(row) - 1) * n:]
    assert int(row[-1]) == sum(int(c) * L ** j for j, c in enumerate(tail))


# ------------------------------------------------------------- quantizer ---
def _f16_groups(rng, shape, scale=1.0):
    return (rng.standard_normal(shape).astype(np.float32) * np.float32(scale)).astype(np.float16)


def _rne(fr: Fraction) -> int:
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


@pytest.mark.parametrize("L,G", [(5, 32), (6, 32), (8, 64), (4, 128), (3, 32)])
def test_quantizer_against_exact_rational(L, G):
    """Codes equal exact-rational round-half-even of (x - z)/s clamped to the
    grid, z is the exact group minimum, s is within one fp16 ulp of the exact
    range/(L-1) (equal to its nearest fp16 in nearly all groups)."""
    rng = np.random.default_rng(100 + L)
    x = _f16_groups(rng, (400, G), scale=3.0)
    x[0] = x[0, 0]                                   # constant group
    x[1, 5] = np.float16(-0.0); x[1, 6] = np.float16(0.0)
    codes, s16, z16 = O.quantize_groups(x, L)
    exact_nearest = 0
    for g in range(x.shape[0]):
        xs = [Fraction(float(v)) for v in x[g]]
        mn, mx = min(xs), max(xs)
        assert Fraction(float(z16[g])) == mn
        s = Fraction(float(s16[g]))
        target = (mx - mn) / (L - 1)
        ulp = Fraction(2) ** (math.frexp(float(max(s, target)) or 1.0)[1] - 11) if target else 0
        assert abs(s - target) <= ulp
        if float(np.float16(float(target))) == float(s16[g]):
            exact_nearest += 1
        for i, xv in enumerate(xs):
            want = 0 if s == 0 else min(max(_rne((xv - mn) / s), 0), L - 1)
            assert codes[g, i] == want, (g, i)
    assert exact_nearest >= x.shape[0] - 2


def test_signed_zero_total_order():
    """-0 sorts below +0 (IEEE total order), whichever comes first."""
    x = np.abs(np.linspace(0.5, 3.0, 32)).astype(np.float16)
    x[3] = np.float16(0.0); x[9] = np.float16(-0.0)
    _, _, z = O.quantize_groups(x[None], 6)
    assert z.view(np.uint16)[0] == 0x8000
    y = -x
    y[3] = np.float16(0.0); y[9] = np.float16(-0.0)
    codes, s, z = O.quantize_groups(y[None], 6)
    assert codes[0, 3] == codes[0, 9] == 5                   # both zeros sit at the top code


def test_top_code_saturates_when_scale_rounds_down():
    """A subnormal fp16 scale can round far below range/(L-1); the top code is
    then clamped to L-1 (the grid has L levels)."""
    x = np.zeros((1, 32), np.float16)
    x[0, 1] = np.float16(7 * 2.0 ** -24)                  # range 7 ulp, s32 = 1.4 ulp -> s = 1 ulp
    codes, s16, z16 = O.quantize_groups(x, 6)
    assert s16.view(np.uint16)[0] == 1
    assert codes[0, 1] == 5 and codes[0, 0] == 0


def _fp16_int(x16):
    """fp16 values as exact integers in units of 2**-24 (every fp16 is one)."""
    b = x16.view(np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    e, m = mag >> 10, mag & 0x3FF
    val = np.where(e == 0, m, (m | 0x400) << np.maximum(e - 1, 0))
    return np.where(b & 0x8000, -val, val)


@pytest.mark.parametrize("L,G", [(5, 32), (6, 32), (8, 64), (3, 32)])
def test_quantizer_codes_exact_integer_bulk(L, G):
    """Millions of values: codes equal round-half-even of the exact quotient
    (x - z)/s computed in integers (all fp16 values are integer multiples of
    2**-24), clamped to the grid."""
    rng = np.random.default_rng(1000 + L)
    x = _f16_groups(rng, ((1 << 22) // G, G))
    x[:, :4] *= np.float16(10)
    codes, s16, z16 = O.quantize_groups(x, L)
    X, Z, S = _fp16_int(x), _fp16_int(z16)[:, None], _fp16_int(s16)[:, None]
    num = X - Z
    assert np.all(num >= 0) and np.all(S > 0)
    q = num // S
    r = num - q * S
    up = (2 * r > S) | ((2 * r == S) & (q % 2 == 1))
    want = np.minimum(q + up, L - 1)
    assert np.array_equal(codes.astype(np.int64), want)


@pytest.mark.parametrize("L,G", [(5, 32), (6, 32), (8, 64), (4, 128), (3, 32)])
def test_quantizer_half_step(L, G):
    """Round-trip error is at most half a step (plus the top-code saturation
    when the fp16 scale rounded down)."""
    rng = np.random.default_rng(7 + L)
    x = _f16_groups(rng, (3000, G))
    x[:, :4] *= np.float16(10)
    codes, s16, z16 = O.quantize_groups(x, L)
    xh = O.dequantize_groups(codes, s16, z16)
    xf = x.astype(np.float64)
    s = s16.astype(np.float64)[:, None]
    rng_ = (xf.max(1) - xf.min(1))[:, None]
    sat = np.maximum(0.0, rng_ - (L - 1) * s)
    assert np.all(np.abs(xh - xf) <= np.maximum(s / 2 * (1 + 2 ** -20), sat + 1e-12))
    assert np.all(sat <= (L - 1) * s * 2 ** -11 + 1e-12)
    assert codes.max() <= L - 1


def test_quantizer_grid_points_and_constant_group():
    for L in (3, 4, 5, 6, 8):
        c = np.arange(L, dtype=np.float32)
        x = (np.float32(-1.0) + c * np.float32(0.25)).astype(np.float16)[None, :]
        codes, s16, z16 = O.quantize_groups(x, L)
        assert float(s16[0]) == 0.25 and float(z16[0]) == -1.0
        assert codes[0].tolist() == list(range(L))
        assert np.array_equal(O.dequantize_groups(codes, s16, z16)[0], x[0].astype(np.float64))
    x = np.full((1, 32), np.float16(1.375))
    codes, s16, z16 = O.quantize_groups(x, 6)
    assert float(s16[0]) == 0.0 and codes.max() == 0
    assert np.all(O.dequantize_groups(codes, s16, z16) == 1.375)


def test_two_bit_textbook_quantizer():
    """L = 4 is the textbook asymmetric 2-bit min/max quantizer: codes
    round((x - min) / ((max - min)/3)) in {0,1,2,3}, min -> 0, max -> 3."""
    rng = np.random.default_rng(3)
    x = _f16_groups(rng, (2000, 32))
    codes, s16, z16 = O.quantize_groups(x, 4)
    xf = x.astype(np.float64)
    assert np.all(codes[np.arange(2000), xf.argmin(1)] == 0)
    assert np.all(codes[np.arange(2000), xf.argmax(1)] == 3)
    ref = np.rint((xf - xf.min(1, keepdims=True)) / ((xf.max(1) - xf.min(1)) / 3)[:, None])
    assert np.mean(codes == ref) > 0.999


# ------------------------------------------------------------------ rank ---
def test_rank_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for T in (1, 2, 17, 300, 2048):
        s = np.exp(rng.standard_normal((2, T)).astype(np.float32)).astype(np.float32)
        if T > 10:
            s[0, 3] = s[0, 7] = s[0, 9]              # ties
            s[1, 1] = np.float32(0.0); s[1, 2] = np.float32(-0.0)   # equal values
            s[1, 4] = s[1, 1]
        r = O.rank_desc(s)
        for b in range(2):
            sb = s[b].astype(np.float64)
            for t in range(T):
                want = int(np.sum(sb > sb[t]) + np.sum(sb[:t] == sb[t]))
                assert r[b, t] == want
            assert sorted(r[b].tolist()) == list(range(T))


def test_tiers_preserve_every_token():
    rng = np.random.default_rng(5)
    B, T, n_hi = 3, 1000, 371
    s = rng.standard_normal((B, T)).astype(np.float32)
    rank = O.rank_desc(s)
    tokmap, counts, inv = O.tiers_and_slots(rank, n_hi)
    for b in range(B):
        assert tuple(counts[b]) == (n_hi, T - n_hi)
        tier = tokmap[b] >> 31
        slot = tokmap[b] & 0x7FFFFFFF
        for p in (0, 1):
            toks = np.nonzero(tier == p)[0]
            assert np.array_equal(slot[toks], np.arange(len(toks)))   # token order
            assert np.array_equal(inv[b][p], toks)
        # the high tier holds exactly the n_hi best scores
        assert s[b][tier == 0].min() >= s[b][tier == 1].max()


# --------------------------------------------------------- running median ---
def test_running_median_against_resort():
    rng = np.random.default_rng(9)
    for n0 in (1, 2, 5, 64):
        pre = np.exp(rng.standard_normal(n0).astype(np.float32))
        rm = O.RunningMedian(pre)
        hist = [float(x) for x in pre]
        for _ in range(40):
            snew = float(np.exp(np.float32(rng.standard_normal())))
            if rng.random() < 0.2:
                snew = hist[rng.integers(len(hist))]          # exact tie with a prior score
            med = float(np.median(np.array(hist, dtype=np.float64)))
            tier = rm.decide_and_insert(snew)
            assert tier == (0 if snew > med else 1)
            hist.append(float(np.float32(snew)))


# ------------------------------------------------------------- attention ---
def _naive_attention(q, k, v, scale):
    out = []
    for qh in q:
        sc = [scale * math.fsum(float(a) * float(b) for a, b in zip(qh, kt)) for kt in k]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        den = math.fsum(w)
        out.append([math.fsum(wi * float(vt[d]) for wi, vt in zip(w, v)) / den for d in range(len(v[0]))])
    return np.array(out)


def test_attention_brute_force_and_closed_forms():
    rng = np.random.default_rng(21)
    Hg, N, D = 4, 9, 16
    q = rng.standard_normal((Hg, D))
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    o = O.attention_fp64(q, k, v, 0.25)
    assert np.allclose(o, _naive_attention(q, k, v, 0.25), rtol=1e-12, atol=1e-13)
    # a single token: output is that token's value
    assert np.allclose(O.attention_fp64(q, k[:1], v[:1], 0.3), np.repeat(v[:1], Hg, 0), rtol=0, atol=1e-15)
    # identical keys: the mean of the values
    kk = np.repeat(k[:1], N, 0)
    assert np.allclose(O.attention_fp64(q, kk, v, 0.3), np.repeat(v.mean(0, keepdims=True), Hg, 0), atol=1e-14)
    # token order does not matter
    perm = rng.permutation(N)
    assert np.allclose(O.attention_fp64(q, k[perm], v[perm], 0.25), o, atol=1e-14)
    # one dominant score selects its row
    k2 = k.copy(); k2[4] = q[0] * 50
    assert np.allclose(O.attention_fp64(q[:1], k2, v, 1.0)[0], v[4], atol=1e-9)


def test_attention_lse_brute_force_and_closed_forms():
    rng = np.random.default_rng(22)
    R, N, D = 6, 11, 16
    q = rng.standard_normal((R, D))
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    o, lse = O.attention_lse_fp64(q, k, v, 0.3)
    # the output rows are plain attention, row by row
    assert np.allclose(o, _naive_attention(q, k, v, 0.3), rtol=1e-12, atol=1e-13)
    # log-sum-exp by brute force: pure-Python sum of exponentials, no shift
    for r in range(R):
        sc = [0.3 * math.fsum(float(q[r, d]) * float(k[t, d]) for d in range(D)) for t in range(N)]
        assert abs(lse[r] - math.log(math.fsum(math.exp(x) for x in sc))) < 1e-12
    # identical keys: lse = score + ln N and the output is the mean value
    kk = np.repeat(k[:1], N, 0)
    o2, lse2 = O.attention_lse_fp64(q, kk, v, 0.3)
    assert np.allclose(lse2, 0.3 * (q @ k[0]) + math.log(N), atol=1e-13)
    assert np.allclose(o2, np.repeat(v.mean(0, keepdims=True), R, 0), atol=1e-14)
    # one token: lse is its score, the output its value
    o3, lse3 = O.attention_lse_fp64(q, k[:1], v[:1], 0.3)
    assert np.allclose(lse3, 0.3 * (q @ k[0]), atol=1e-14)
    assert np.allclose(o3, np.repeat(v[:1], R, 0), atol=1e-15)
    # huge scores do not overflow (the shift by the row maximum)
    o4, lse4 = O.attention_lse_fp64(q * 1e3, k, v, 1.0)
    assert np.all(np.isfinite(lse4)) and np.all(np.isfinite(o4))
    # splitting the keys in two and merging by log-sum-exp gives the whole
    oa, la = O.attention_lse_fp64(q, k[:5], v[:5], 0.3)
    ob, lb = O.attention_lse_fp64(q, k[5:], v[5:], 0.3)
    lm = np.logaddexp(la, lb)
    om = oa * np.exp(la - lm)[:, None] + ob * np.exp(lb - lm)[:, None]
    assert np.allclose(lm, lse, atol=1e-13) and np.allclose(om, o, atol=1e-13)


def test_token_attention_mass_pins():
    rng = np.random.default_rng(23)
    Hq, Hkv, N, D = 8, 2, 13, 16
    q = rng.standard_normal((Hq, D))
    ks = [rng.standard_normal((N, D)) for _ in range(Hkv)]
    m = O.token_attention_mass(q, ks, 0.3)
    # every head's weights sum to one
    assert abs(m.sum() - Hq) < 1e-12 and np.all(m >= 0)
    # brute force: pure-Python softmax of every head
    for t in (0, 5, 12):
        tot = 0.0
        for hq in range(Hq):
            sc = [0.3 * math.fsum(float(q[hq, d]) * float(ks[hq // 4][u, d]) for d in range(D)) for u in range(N)]
            den = math.fsum(math.exp(x) for x in sc)
            tot += math.exp(sc[t]) / den
        assert abs(m[t] - tot) < 1e-12
    # identical keys: every token gets Hq / N; one token gets Hq
    same = [np.repeat(k[:1], N, 0) for k in ks]
    assert np.allclose(O.token_attention_mass(q, same, 0.3), Hq / N, atol=1e-14)
    assert np.allclose(O.token_attention_mass(q, [k[:1] for k in ks], 0.3), [Hq], atol=1e-14)
    # it agrees with the weights behind attention_lse_fp64 (exp(s - lse))
    _, lse = O.attention_lse_fp64(q[:4], ks[0], ks[0], 0.3)
    w = np.exp(0.3 * (q[:4] @ ks[0].T) - lse[:, None]).sum(0)
    _, lse2 = O.attention_lse_fp64(q[4:], ks[1], ks[1], 0.3)
    w += np.exp(0.3 * (q[4:] @ ks[1].T) - lse2[:, None]).sum(0)
    assert np.allclose(w, m, atol=1e-13)


def test_row_rel_err_definition():
    r = np.array([[1.0, -2.0, 0.5]])
    o = np.array([[1.0, -2.002, 0.5]])
    assert abs(O.row_rel_err(o, r) - 0.001) < 1e-12


# ------------------------------------------------------------ tiered unit ---
def test_tiered_unit_roundtrip_small():
    w = synth.W_SINGLE.shrink(tokens=300, name="tiny")
    inp = synth.make_inputs(w)
    rank = O.rank_desc(inp.scores)
    tokmap, counts, inv = O.tiers_and_slots(rank, w.n_hi)
    hi, lo = O.quantize_tiered_unit(inp.k[0, :, 0], inp.v[0, :, 0], inv[0], 6, 5, 32)
    assert hi.n + lo.n == 300 and hi.n == 150
    # pool rows are the tier's tokens in token order, within half a step
    for pool, toks in ((hi, inv[0][0]), (lo, inv[0][1])):
        kh = pool.k_hat()
        ks = np.repeat(pool.k_scale.astype(np.float64), 32, axis=1)
        assert np.all(np.abs(kh - inp.k[0, toks, 0].astype(np.float64)) <= ks / 2 * (1 + 1e-6) + 1e-12)
        vw = pool.v_words()
        n = O.codes_per_word(pool.L)
        assert vw.shape == (-(-pool.n // n), 128)
        assert np.array_equal(O.unpack_digits(vw, pool.L, n).transpose(0, 2, 1).reshape(-1, 128)[:pool.n],
                              pool.v_codes)


# ----------------------------------------------------------------- kchan ---
def test_kchan_unit_structure():
    w = synth.W_KCHAN.shrink(tokens=128 * 3 + 50, batch=1, kv_heads=1, q_heads=4, name="tiny5")
    inp = synth.make_inputs(w)
    k, v = inp.k[0, :, 0], inp.v[0, :, 0]
    u = O.KChanUnit(k, v, w)
    assert u.n_q == 256 and u.k_win.shape[0] == 178            # 2 blocks + window of 178
    assert np.array_equal(u.k_win, k[256:]) and np.array_equal(u.v_win, v[256:])
    mag = np.abs(k[:256].astype(np.float64))
    for t in range(256):
        top = sorted(range(128), key=lambda d: (-mag[t, d], d))[:2]
        assert u.sp_ch[t].tolist() == sorted(top)
        assert np.array_equal(u.sp_val[t], k[t, sorted(top)])
    kh = u.k_hat()[:256]
    step = np.repeat(u.k_scale.astype(np.float64)[:, None, :], 128, axis=1).reshape(256, 128)
    assert np.all(np.abs(kh - k[:256].astype(np.float64)) <= step / 2 * (1 + 1e-6) + 1e-12)
    # outlier channels are mostly taken by the sparse list
    assert np.mean(u.sp_ch < 4) > 0.9
    vh = u.v_hat()
    assert np.array_equal(vh[256:], v[256:].astype(np.float64))


@pytest.mark.parametrize("kl,vl,vg,n_vl", [(4, 3, 32, 20), (3, 5, 64, 13), (8, 6, 128, 12)])
def test_kchan_unit_value_half(kl, vl, vg, n_vl):
    """The value half of a per-channel-key unit: values are quantized per
    token in groups of v_group consecutive channels at v_levels (not at the
    key levels, not per channel), with the exact group minimum as zero, the
    scale within one fp16 ulp of the exact range / (v_levels - 1), codes
    the exact round-half-even of (x - z) / s on the grid; the column words
    unpack, n_vl digits each (worked by hand: 3^20, 5^13 and 6^12 are the
    largest powers at most 2^32), back to the codes along the slot axis; the
    dequantized values are z + c s and within half a step of the input."""
    w = synth.W_KCHAN.shrink(tokens=128 * 3 + 50, batch=1, kv_heads=1, q_heads=4, name="tiny5v",
                             k_levels=kl, v_levels=vl, v_group=vg)
    inp = synth.make_inputs(w)
    k, v = inp.k[0, :, 0], inp.v[0, :, 0]
    v = v.copy()
    v[3, :vg] = np.float16(0.625)                                # a constant group
    v[7, 1] = np.float16(-0.0); v[7, 2] = np.float16(0.0)
    u = O.KChanUnit(k, v, w)
    nq, ng = u.n_q, 128 // vg
    assert nq == 256
    assert u.v_scale.shape == (nq, ng) and u.v_zero.shape == (nq, ng) and u.v_codes.shape == (nq, 128)
    assert int(u.v_codes.max()) == vl - 1 and vl != kl
    for t in range(nq):
        for g in range(ng):
            xs = [Fraction(float(x)) for x in v[t, g * vg:(g + 1) * vg]]
            mn, mx = min(xs), max(xs)
            assert Fraction(float(u.v_zero[t, g])) == mn
            s = Fraction(float(u.v_scale[t, g]))
            target = (mx - mn) / (vl - 1)
            ulp = Fraction(2) ** (math.frexp(float(max(s, target)) or 1.0)[1] - 11) if target else 0
            assert abs(s - target) <= ulp, (t, g)
            for i, xv in enumerate(xs):
                want = 0 if s == 0 else min(max(_rne((xv - mn) / s), 0), vl - 1)
                assert u.v_codes[t, g * vg + i] == want, (t, g, i)
    words = u.v_words()
    assert words.shape == (-(-nq // n_vl), 128)
    digits = O.unpack_digits(words, vl, n_vl)                    # [row][channel][digit]
    assert np.array_equal(digits.transpose(0, 2, 1).reshape(-1, 128)[:nq], u.v_codes)
    assert not digits.transpose(0, 2, 1).reshape(-1, 128)[nq:].any()
    vh = u.v_hat()[:nq]
    step = np.repeat(u.v_scale.astype(np.float64), vg, axis=1)
    zero = np.repeat(u.v_zero.astype(np.float64), vg, axis=1)
    assert np.array_equal(vh, zero + u.v_codes.astype(np.float64) * step)
    assert np.all(np.abs(vh - v[:nq].astype(np.float64)) <= step / 2 * (1 + 2.0 ** -20) + 1e-12)
    assert np.array_equal(u.v_hat()[nq:], v[nq:].astype(np.float64))


# ------------------------------------------------------- pre-RoPE keys ---
# KVQuant summary, "techniques" (Pre-RoPE Key Quantization).  The pins fix
# the rotation by what any rotary embedding must satisfy plus quarter turns
# whose images are exact, without restating the formula.

def test_rope_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 128))
    assert np.array_equal(O.rope_rotate(x, np.zeros(50), 10000.0), x)
    y = O.rope_rotate(x, rng.integers(0, 131072, 50), 500000.0)
    pairs = lambda z: np.hypot(z[:, 0::2], z[:, 1::2])           # noqa: E731
    assert np.allclose(pairs(y), pairs(x), rtol=1e-13, atol=0)
    assert not np.allclose(y, x)


def test_rope_quarter_turns_fix_direction_pairing_and_frequencies():
    """Pair 0 turns at rate 1, pair i at base^(-2i/D): (1, 0) in pair 0 at
    position pi/2, and in pair 1 (D = 4, base 10^4: rate 10^-2) at 50 pi,
    becomes (0, 1) -- counterclockwise, within its own adjacent pair; a
    half turn maps it to (-1, 0)."""
    e0 = np.array([[1.0, 0.0, 0.0, 0.0]])
    e2 = np.array([[0.0, 0.0, 1.0, 0.0]])
    assert np.allclose(O.rope_rotate(e0, [math.pi / 2], 1e4), [[0, 1, 0, 0]], atol=1e-15)
    assert np.allclose(O.rope_rotate(e2, [50 * math.pi], 1e4), [[0, 0, 0, 1]], atol=1e-13)
    assert np.allclose(O.rope_rotate(e2, [100 * math.pi], 1e4), [[0, 0, -1, 0]], atol=1e-13)
    # pair 0 is untouched by pair 1's quarter turn position and vice versa
    assert np.allclose(O.rope_rotate(e0, [2 * math.pi], 1e4), e0, atol=1e-14)
    th = O.rope_thetas(128, 500000.0)
    assert th[0] == 1.0 and abs(th[-1] - 500000.0 ** (-126 / 128)) < 1e-20 and np.all(np.diff(th) < 0)


def test_rope_composes_and_scores_depend_on_relative_position():
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal((2, 30, 128))
    a, b = rng.integers(0, 40000, 30), rng.integers(0, 40000, 30)
    ab = O.rope_rotate(O.rope_rotate(k, a, 1e4), b, 1e4)
    assert np.allclose(ab, O.rope_rotate(k, a + b, 1e4), rtol=0, atol=1e-10)
    m, n, sh = rng.integers(0, 60000, 30), rng.integers(0, 60000, 30), rng.integers(0, 60000, 30)
    s1 = np.einsum("td,td->t", O.rope_rotate(q, m, 5e5), O.rope_rotate(k, n, 5e5))
    s2 = np.einsum("td,td->t", O.rope_rotate(q, m + sh, 5e5), O.rope_rotate(k, n + sh, 5e5))
    s3 = np.einsum("td,td->t", q, O.rope_rotate(k, n - m, 5e5))
    assert np.allclose(s1, s2, rtol=0, atol=1e-9) and np.allclose(s1, s3, rtol=0, atol=1e-9)


# --------------------------------------------------------------- storage ---
def test_storage_ratio_closed_forms():
    """Layout bytes per (sequence, KV head), worked by hand for the 32768-token
    6/5-level G=32 unit and the 65536-token kchan unit."""
    D = 128
    # 16384 hi tokens: 11 key words (44 B), ceil(16384/12) = 1366 value word rows
    # of 128 words, 4 groups x 4 B (scale, zero) for K and for V.
    hi = 16384 * 44 + 1366 * 512 + 2 * 16384 * 16
    lo = 16384 * 40 + 1261 * 512 + 2 * 16384 * 16
    assert O.tiered_unit_bytes(16384, 16384, 6, 5, 32, D) == hi + lo
    fp16 = 32768 * 128 * 2 * 2
    assert abs(O.storage_ratio(fp16, hi + lo) - 16777216 / 3769856) < 1e-12
    w = synth.W_KCHAN
    nq = 65408
    b = nq * 32 + 511 * 512 + nq * 8 + (-(-nq // 20)) * 512 + nq * 16 + 128 * 512
    assert O.kchan_unit_bytes(65536, w, D) == b
    assert 5.5 < O.storage_ratio(65536 * 512, b) < 6.0


# ------------------------------------------- channel order and clipping ---
def test_clip_worked_examples():
    """Hand-worked clipped groups (fixture cites SKVQ, Abstract)."""
    rows = _golden("skvq_clip_examples.txt")
    assert len(rows) == 4
    for r in rows:
        clip, L, scale, zero, n = float(r[0]), int(r[1]), float(r[2]), float(r[3]), int(r[4])
        x = np.array([float(t) for t in r[5:5 + n]], dtype=np.float16)
        want = [int(t) for t in r[5 + n:5 + 2 * n]]
        c, s, z = O.quantize_groups(x[None, :], L, clip)
        assert c[0].tolist() == want, (r, c)
        assert float(s[0]) == scale and float(z[0]) == zero


def test_clip_one_is_the_plain_quantizer():
    rng = np.random.default_rng(11)
    x = _f16_groups(rng, (400, 4, 32), 3.0)
    for L in (3, 5, 6, 8):
        a = O.quantize_groups(x, L)
        b = O.quantize_groups(x, L, 1.0)
        for u, v in zip(a, b):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("clip", [0.5, 0.8, 0.95])
def test_clip_codes_are_the_nearest_clipped_grid_point(clip):
    """Brute force: every code is the grid point z + c s (c in 0..L-1) nearest
    to x, with z and s formed from the clipped min and max worked out here in
    exact arithmetic; values beyond the clipped range take the end codes."""
    rng = np.random.default_rng(int(clip * 100))
    x = _f16_groups(rng, (300, 32), 2.0)
    x[::7, 3] = np.float16(25.0)                       # a heavy tail in some groups
    for L in (3, 5, 8):
        c, s, z = O.quantize_groups(x, L, clip)
        for g in range(x.shape[0]):
            xs = [Fraction(float(t)) for t in x[g]]
            lo = Fraction(float(np.float16(np.float32(min(xs)) * np.float32(clip))))
            hi = Fraction(float(np.float16(np.float32(max(xs)) * np.float32(clip))))
            assert Fraction(float(z[g])) == lo
            sf = Fraction(float(s[g]))
            assert abs(sf - (hi - lo) / (L - 1)) <= sf * Fraction(1, 1024) + Fraction(1, 2 ** 24)
            if sf == 0:
                assert not c[g].any()
                continue
            for xi, ci in zip(xs, c[g].tolist()):
                errs = [abs(xi - (lo + k * sf)) for k in range(L)]
                assert errs[ci] <= min(errs) + sf * Fraction(1, 10 ** 5), (g, xi, ci)


def _lossless_pattern(D=128):
    """Rows whose channel d holds a value that depends only on d % 4 (keys)
    or (d // 2) % 4 (values): grouped by that key every group of 32 is
    constant, so a stored order that sorts by it quantizes without loss.
    Neither order is its own inverse, so applying one backwards is caught."""
    kd, vd = np.arange(D) % 4, (np.arange(D) // 2) % 4
    k = np.stack([(kd * (r + 1) - 3).astype(np.float16) for r in range(5)])
    v = np.stack([(vd * 0.5 * (r + 1) + 1).astype(np.float16) for r in range(5)])
    order_k = np.argsort(kd, kind="stable")
    order_v = np.argsort(vd, kind="stable")
    return k, v, order_k, order_v


def test_channel_order_that_makes_groups_constant_is_lossless():
    """SKVQ, Abstract: rearranging channels makes each quantization group's
    channels alike.  In the extreme case every group is constant, the scale
    is 0 and the reconstruction is exact, in the original channel order."""
    k, v, ok, ov = _lossless_pattern()
    p = O.Pool(3, 32, 128, ok, ov)
    p.add_rows(k, v)
    assert np.array_equal(p.k_hat(), k.astype(np.float64))
    assert np.array_equal(p.v_hat(), v.astype(np.float64))
    assert not p.k_scale.astype(np.float64).any() and not p.v_scale.astype(np.float64).any()
    # the stored codes follow the order: position p holds channel order[p]
    assert np.array_equal(p.k_zero[:, 1].astype(np.float64), k[:, ok[32]].astype(np.float64))
    # the natural order and the inverse order both lose information
    for a, b in ((None, None), (np.argsort(ok), np.argsort(ov))):
        q = O.Pool(3, 32, 128, a, b)
        q.add_rows(k, v)
        assert not np.array_equal(q.k_hat(), k.astype(np.float64))
        assert not np.array_equal(q.v_hat(), v.astype(np.float64))


def test_lossless_order_gives_plain_attention():
    """With a lossless order the oracle's attention over the pool equals plain
    attention over the raw rows (original channel order throughout)."""
    k, v, ok, ov = _lossless_pattern()
    p = O.Pool(3, 32, 128, ok, ov)
    p.add_rows(k, v)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 128))
    scale = 1 / math.sqrt(128)
    got = O.attention_fp64(q, p.k_hat(), p.v_hat(), scale)
    ref = _naive_attention(q, k.astype(np.float64), v.astype(np.float64), scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_channel_order_and_clip_lower_key_error_on_spread_outliers():
    """The workload with one outlier key channel per group: its stored order
    gathers the four outliers into the first stored group, so the 96 channels
    stored in the other three groups no longer share a range with an outlier
    and their key reconstruction error falls by more than half (the group
    range shrinks from about one outlier to about two standard deviations
    either side); clipping at 0.9 on these Gaussian groups lowers it further."""
    w = synth.W_SKVQ.shrink(tokens=256, batch=1, kv_heads=1, q_heads=4, name="tiny_skvq")
    inp = synth.make_inputs(w)
    orders = synth.channel_orders(w)
    k, v = inp.k[0, :, 0], inp.v[0, :, 0]
    plain = O.Pool(6, 32, 128)
    plain.add_rows(k, v)
    skvq = O.Pool(6, 32, 128, orders[0, 0], orders[1, 0], w.clip)
    skvq.add_rows(k, v)
    normal = orders[0, 0, 32:]                         # channels stored outside the first group
    assert not np.isin(normal, np.arange(4) * 32).any()
    e_plain = np.abs(plain.k_hat() - k.astype(np.float64))[:, normal].mean()
    e_skvq = np.abs(skvq.k_hat() - k.astype(np.float64))[:, normal].mean()
    assert e_skvq < e_plain / 2, (e_plain, e_skvq)
    unclipped = O.Pool(6, 32, 128, orders[0, 0], orders[1, 0])
    unclipped.add_rows(k, v)
    e_unclipped = np.abs(unclipped.k_hat() - k.astype(np.float64))[:, normal].mean()
    assert e_skvq < e_unclipped, (e_unclipped, e_skvq)
