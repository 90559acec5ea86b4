"""GPU parity of pre-RoPE keys (KVQuant summary, "techniques"): keys are
quantized and stored before the rotary embedding, and the decode turns every
dequantized key by its token position before the dot product.  The stored
cache is the plain one bit for bit (the rotation only happens in decode);
the slot positions equal the tier split's slot -> token map; attention and
the token mass are checked against the oracle, which turns the fp64
dequantized keys with ``rope_rotate``."""
import numpy as np
import pytest

from mixed_precision_kv_amd import kvq, synth
from oracle import kvq_oracle as O
import layout_view as LV
from gpu_harness import GpuRun, TOL, compare_tiered_unit, log, oracle_tiers, oracle_unit

pytestmark = pytest.mark.gpu


def _keys(w, pools, pos):
    """Rotated dequantized keys of one unit, pools concatenated (hi, lo)."""
    return np.concatenate([O.rope_rotate(p.k_hat(), np.asarray(ps[:p.n]), w.rope_theta)
                           for p, ps in zip(pools, pos)])


def _decode_err(w, run, q, pools, pos, units=None, max_len=None, plain_too=False):
    out = run.decode(q, max_len)
    g = w.q_heads // w.kv_heads
    errs, gaps = [], []
    for b in range(w.batch):
        for h in range(w.kv_heads):
            if units is not None and b * w.kv_heads + h not in units:
                continue
            pl = pools[(b, h)]
            vh = np.concatenate([p.v_hat() for p in pl])
            qb = q[b, h * g:(h + 1) * g].astype(np.float64)
            ref = O.decode_unit(qb, _keys(w, pl, pos[b]), vh, float(run.scale))
            errs.append(O.row_rel_err(out[b, h * g:(h + 1) * g], ref))
            if plain_too:
                kp = np.concatenate([p.k_hat() for p in pl])
                gaps.append(O.row_rel_err(O.decode_unit(qb, kp, vh, float(run.scale)), ref))
    return max(errs), (min(gaps) if gaps else None)


@pytest.mark.parametrize("lh,ll,g,T", [(6, 5, 32, 1999), (8, 6, 64, 3001), (4, 3, 128, 1201), (7, 5, 32, 777),
                                        (5, 7, 64, 1500)])
def test_rope_quantize_and_decode(lh, ll, g, T):
    w = synth.W_ROPE.shrink(name=f"rope_{lh}_{ll}_g{g}_T{T}", batch=2, kv_heads=2, q_heads=8, tokens=T,
                            levels_hi=lh, levels_lo=ll, group=g)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _, _, _, inv = oracle_tiers(w, inp)
    buf = run.buf()
    pools = {}
    for b in range(w.batch):
        for p in range(2):
            assert np.array_equal(LV.slot_positions(buf, run.lay, p)[b, :len(inv[b][p])], inv[b][p]), "positions"
        for h in range(w.kv_heads):
            pools[(b, h)] = oracle_unit(w, inp, inv, b, h)
            compare_tiered_unit(buf, run.lay, pools[(b, h)], b * w.kv_heads + h, w.name)
    pos = [[inv[b][0], inv[b][1]] for b in range(w.batch)]
    err, gap = _decode_err(w, run, inp.q, pools, pos, plain_too=True)
    log(f"{w.name}: max row rel err {err:.3e} (unrotated keys would be {gap:.2e} off)")
    assert err <= TOL and gap > 50 * TOL


def test_rope_appends_and_token_mass():
    """Generation steps: appended tokens sit at positions T, T + 1, ...; the
    decode after each step and the token mass at the end."""
    w = synth.W_APPEND.shrink(name="rope_append", batch=3, kv_heads=2, q_heads=8, tokens=300, append_steps=24,
                              rope_theta=10000.0)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _, tokmap, _, inv = oracle_tiers(w, inp)
    med = [O.RunningMedian(inp.scores[b]) for b in range(w.batch)]
    pools = {(b, h): oracle_unit(w, inp, inv, b, h) for b in range(w.batch) for h in range(w.kv_heads)}
    pos = [[list(inv[b][0]), list(inv[b][1])] for b in range(w.batch)]
    for i, st in enumerate(inp.steps):
        run.append(st)
        for b in range(w.batch):
            tier = med[b].decide_and_insert(st["score_new"][b])
            pos[b][tier].append(w.tokens + i)
            for h in range(w.kv_heads):
                pools[(b, h)][tier].add_rows(st["k_new"][b, h][None], st["v_new"][b, h][None])
        if i % 6 == 5:
            err, _ = _decode_err(w, run, st["q"], pools, pos, max_len=w.tokens + i + 1)
            log(f"step {i}: max row rel err {err:.3e}")
            assert err <= TOL, f"step {i}"
    buf = run.buf()
    for b in range(w.batch):
        for p in range(2):
            assert np.array_equal(LV.slot_positions(buf, run.lay, p)[b, :len(pos[b][p])], pos[b][p])
    q = inp.steps[-1]["q"]
    mass = run.decode_mass(q)
    n = w.capacity
    for b in range(w.batch):
        ks = []
        for h in range(w.kv_heads):
            kt = np.zeros((n, w.head_dim))
            for p in range(2):
                kt[np.asarray(pos[b][p], dtype=np.int64)] = O.rope_rotate(
                    pools[(b, h)][p].k_hat(), np.asarray(pos[b][p]), w.rope_theta)
            ks.append(kt)
        ref = O.token_attention_mass(q[b].astype(np.float64), ks, float(run.scale))
        got = mass[b, :n].astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1e-4 * ref + 1e-6), f"token mass b{b}"


@pytest.mark.parametrize("w", [synth.W_ROPE, synth.W_ROPE_LONG], ids=lambda w: w.name)
def test_rope_fullsize(w):
    """The Llama-shaped layer and the 131072-token workload with pre-RoPE
    keys, in the bench's launch configuration: sampled units."""
    log(f"case {w.name} full size")
    inp = synth.make_inputs(w, steps=0)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _, _, _, inv = oracle_tiers(w, inp)
    U = w.batch * w.kv_heads
    units = sorted({0, U // 2 + 1 if U > 2 else U - 1, U - 1})
    buf = run.buf()
    pools = {}
    for u in units:
        b, h = divmod(u, w.kv_heads)
        pools[(b, h)] = oracle_unit(w, inp, inv, b, h)
        compare_tiered_unit(buf, run.lay, pools[(b, h)], u, w.name)
    pos = [[inv[b][0], inv[b][1]] for b in range(w.batch)]
    err, gap = _decode_err(w, run, inp.q, pools, pos, units=units, plain_too=True)
    log(f"{w.name}: units {units} max row rel err {err:.3e} (unrotated keys {gap:.2e} off)")
    assert err <= TOL and gap > 50 * TOL
