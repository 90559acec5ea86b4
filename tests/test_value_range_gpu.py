"""GPU parity with large value ranges.

The decode kernels form the fp16 product 2^6 p * s of a softmax weight and a
value group scale.  Scales just under 1024 take that product unscaled; a
sequence that stores a larger value scale is flagged (bit 1 of its
counters[b][3]) and decode scales its value operand down.  These cases scale
the values of chosen sequences (in fp32, recast to fp16; the oracle and the
GPU read the same bytes) so that the largest value scale lands just under
1024 or far above it, and check codes, flags, decode, multi-query attention
and the token mass against the oracle."""
import numpy as np
import pytest

from mixed_precision_kv_amd import synth
from oracle import kvq_oracle as O
import layout_view as LV
from gpu_harness import GpuRun, TOL, check_kchan, check_tiered, log, oracle_tiers, oracle_unit

pytestmark = pytest.mark.gpu


def _scale_values(v, seqs, lmin, group, target):
    """Values of sequences `seqs` multiplied by one fp32 factor so that the
    largest group range / (lmin - 1) of the input is `target`."""
    v = v.copy()
    for b in seqs:
        x = v[b].astype(np.float32)
        g = x.reshape(x.shape[0], x.shape[1], -1, group)
        rng = float((g.max(axis=-1) - g.min(axis=-1)).max())
        f = np.float32(target * (lmin - 1) / rng)
        v[b] = (x * f).astype(np.float16)
    assert np.all(np.isfinite(v))
    return v


@pytest.mark.parametrize("lh,ll,g,target,seqs", [
    (8, 6, 64, 1000.0, (0, 1)),      # just under: no flag, operand unscaled
    (4, 5, 32, 1000.0, (0, 1)),
    (6, 4, 128, 1010.0, (0, 1)),
    (8, 6, 64, 8000.0, (0,)),        # far above in sequence 0 only
    (4, 5, 32, 5000.0, (1,)),
    (6, 4, 128, 9000.0, (0, 1)),
])
def test_tiered_large_value_scales(lh, ll, g, target, seqs):
    w = synth.W_LLAMA.shrink(name=f"vrange_{lh}_{ll}_g{g}_{int(target)}", batch=2, kv_heads=2, q_heads=8,
                             tokens=1201, levels_hi=lh, levels_lo=ll, group=g)
    log(f"case {w.name} seqs {seqs}")
    inp = synth.make_inputs(w)
    inp.v = _scale_values(inp.v, seqs, min(lh, ll), g, target)
    run = GpuRun(w, inp)
    run.quantize()
    check_tiered(w, inp, run)                         # words, scales, attention vs the oracle

    # the flag: set exactly for the sequences that store a value scale >= 1024
    _, _, _, inv = oracle_tiers(w, inp)
    big = []
    for b in range(w.batch):
        smax = max(float(p.v_scale.astype(np.float32).max()) for h in range(w.kv_heads)
                   for p in oracle_unit(w, inp, inv, b, h))
        big.append(smax >= 1024.0)
    flags = LV.counters(run.buf(), run.lay)[:, 3]
    log(f"flags {flags.tolist()} expected big {big}")
    assert [(int(f) >> 1) & 1 for f in flags] == [int(x) for x in big]
    assert not (flags & 1).any()
    if target < 1024.0:
        assert not any(big)

    # multi-query attention over the same cache
    M = 5
    qm = synth.make_queries(w, M)
    out, lse = run.decode_multi(qm)
    gq = w.q_heads // w.kv_heads
    errs, lerrs = [], []
    for b in range(w.batch):
        for h in range(w.kv_heads):
            pools = oracle_unit(w, inp, inv, b, h)
            kh = np.concatenate([p.k_hat() for p in pools])
            vh = np.concatenate([p.v_hat() for p in pools])
            qr = qm[b, :, h * gq:(h + 1) * gq].reshape(M * gq, -1).astype(np.float64)
            ref, lref = O.attention_lse_fp64(qr, kh, vh, float(run.scale))
            errs.append(O.row_rel_err(out[b, :, h * gq:(h + 1) * gq].reshape(M * gq, -1), ref))
            lerrs.append(float(np.abs(lse[b, :, h * gq:(h + 1) * gq].reshape(-1) - lref).max()))
    log(f"multi-query: max row rel err {max(errs):.3e}, lse {max(lerrs):.2e}")
    assert max(errs) <= TOL and max(lerrs) <= 1e-4

    # the token mass comes out of the same decode
    mass = run.decode_mass(inp.q)
    _, tokmap, _, _ = oracle_tiers(w, inp)
    for b in range(w.batch):
        ks = []
        for h in range(w.kv_heads):
            pools = oracle_unit(w, inp, inv, b, h)
            kh = np.concatenate([p.k_hat() for p in pools])
            slot = (tokmap[b] & 0x7FFFFFFF).astype(np.int64)
            lo = (tokmap[b] >> 31).astype(bool)
            ks.append(kh[np.where(lo, pools[0].n + slot, slot)])
        ref = O.token_attention_mass(inp.q[b].astype(np.float64), ks, float(run.scale))
        got = mass[b, :w.tokens].astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1e-4 * ref + 1e-6), f"token mass b{b}"
        assert not mass[b, w.tokens:].any()


@pytest.mark.parametrize("target,seqs", [(1000.0, (0, 1)), (12000.0, (1,))])
def test_kchan_large_value_scales(target, seqs):
    """Per-channel-key cache (3-level values, groups of 32): the matrix-core
    decode with value scales under and far above 1024."""
    w = synth.W_KCHAN.shrink(name=f"kchan_vrange_{int(target)}", batch=2, kv_heads=2, q_heads=8, tokens=1408)
    log(f"case {w.name} seqs {seqs}")
    inp = synth.make_inputs(w)
    inp.v = _scale_values(inp.v, seqs, w.v_levels, w.v_group, target)
    run = GpuRun(w, inp)
    run.quantize()
    check_kchan(w, inp, run)
    big = []
    for b in range(w.batch):
        smax = max(float(O.KChanUnit(inp.k[b, :, h], inp.v[b, :, h], w).v_scale.astype(np.float32).max())
                   for h in range(w.kv_heads))
        big.append(smax >= 1024.0)
    flags = LV.counters(run.buf(), run.lay)[:, 3]
    log(f"flags {flags.tolist()} expected big {big}")
    assert [(int(f) >> 1) & 1 for f in flags] == [int(x) for x in big]


def test_append_flags_large_value_scale():
    """An appended token whose value scale is 1024 or more flags its
    sequence; decode after it still matches the oracle."""
    w = synth.W_APPEND.shrink(name="append_vrange", batch=2, kv_heads=2, q_heads=8, tokens=300, append_steps=3)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    assert not (LV.counters(run.buf(), run.lay)[:, 3]).any()
    _, _, _, inv = oracle_tiers(w, inp)
    meds = [O.RunningMedian(inp.scores[b]) for b in range(w.batch)]
    pools = [[oracle_unit(w, inp, inv, b, h) for h in range(w.kv_heads)] for b in range(w.batch)]
    for i, st in enumerate(inp.steps):
        st = dict(st)
        if i == 1:
            v = st["v_new"].astype(np.float32).copy()
            v[1] *= np.float32(3000.0)                   # sequence 1: scales far above 1024
            st["v_new"] = v.astype(np.float16)
        run.append(st)
        for b in range(w.batch):
            tier = meds[b].decide_and_insert(float(st["score_new"][b]))
            for h in range(w.kv_heads):
                pools[b][h][tier].add_rows(st["k_new"][b, h][None], st["v_new"][b, h][None])
    flags = LV.counters(run.buf(), run.lay)[:, 3]
    log(f"flags {flags.tolist()}")
    assert flags.tolist() == [0, 2]
    q = inp.steps[-1]["q"]
    out = run.decode(q, max_len=w.capacity)
    gq = w.q_heads // w.kv_heads
    errs = []
    for b in range(w.batch):
        for h in range(w.kv_heads):
            kh = np.concatenate([p.k_hat() for p in pools[b][h]])
            vh = np.concatenate([p.v_hat() for p in pools[b][h]])
            ref = O.decode_unit(q[b, h * gq:(h + 1) * gq].astype(np.float64), kh, vh, float(run.scale))
            errs.append(O.row_rel_err(out[b, h * gq:(h + 1) * gq], ref))
    log(f"{w.name}: max row rel err {max(errs):.3e}")
    assert max(errs) <= TOL
