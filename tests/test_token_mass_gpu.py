"""GPU parity of the per-token attention mass that decode reports
(kvq_decode_attn_mass): every cached token's softmax weight summed over the
sequence's query heads, against the oracle in fp64, plus the decode output.

Tolerance: |mass - ref| <= 1e-4 * ref + 1e-6 per token.  A token's weight is
exp(s - lse) with s and lse carrying fp32 rounding of a dot product and a
sum (about 1e-6 relative on scores of order 10, so about 1e-5 on the
weight); summing 4 Hkv heads adds nothing of that order.  The sum over
tokens must be Hq to 1e-4 relative."""
import numpy as np
import pytest

from mixed_precision_kv_amd import kvq, synth
from oracle import kvq_oracle as O
from gpu_harness import (GpuRun, TOL, keys_in_token_order, log, mass_mismatches, oracle_tiers, oracle_unit,
                         oracle_unit_attention, to_dev)

pytestmark = pytest.mark.gpu


def _decode_mass(run, q_np, max_len):
    import torch
    ws = torch.empty(kvq.workspace_bytes(run.lay, kvq.OP_DECODE_MASS, run.w.capacity), dtype=torch.uint8,
                     device=run.cache.device)
    q = to_dev(q_np)
    out = torch.empty_like(q)
    mass = torch.full((run.w.batch, max_len), float("nan"), dtype=torch.float32, device=run.cache.device)
    kvq.decode_attn_mass(run.lay, run.cache, q, float(run.scale), max_len, out, mass, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), mass.cpu().numpy()


def _check(w, inp, run, q, n, pools, inv, max_len):
    out, mass = _decode_mass(run, q, max_len)
    g = w.q_heads // w.kv_heads
    errs = []
    for b in range(w.batch):
        ks = [keys_in_token_order(pools[(b, h)], inv[b], n) for h in range(w.kv_heads)]
        ref = O.token_attention_mass(q[b].astype(np.float64), ks, float(run.scale))
        got = mass[b, :n].astype(np.float64)
        bad = mass_mismatches(got, ref)
        assert not bad.any(), f"b{b}: {int(bad.sum())} tokens, worst {np.abs(got - ref).max():.3e}"
        assert abs(got.sum() - w.q_heads) <= 1e-4 * w.q_heads
        assert np.all(mass[b, n:] == 0.0)
        for h in range(w.kv_heads):
            p = pools[(b, h)]
            kh = np.concatenate([p[0].k_hat(), p[1].k_hat()])
            vh = np.concatenate([p[0].v_hat(), p[1].v_hat()])
            ref_o = oracle_unit_attention(w, q, b, h, kh, vh, run.scale)
            errs.append(O.row_rel_err(out[b, h * g:(h + 1) * g], ref_o))
    assert max(errs) <= TOL
    return mass


def _setup(w):
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _, _, _, inv = oracle_tiers(w, inp)
    pools = {(b, h): oracle_unit(w, inp, inv, b, h)
             for b in range(w.batch) for h in range(w.kv_heads)}
    inv = [[list(inv[b][0]), list(inv[b][1])] for b in range(w.batch)]
    return inp, run, pools, inv


@pytest.mark.parametrize("lh,ll,g,T", [(6, 5, 32, 1999), (8, 6, 64, 3001), (4, 3, 128, 1201), (8, 7, 32, 1)])
def test_token_mass_after_quantize(lh, ll, g, T):
    w = synth.W_LLAMA.shrink(name=f"mass_{lh}_{ll}_g{g}_T{T}", batch=2, kv_heads=2, q_heads=8, tokens=T,
                    levels_hi=lh, levels_lo=ll, group=g)
    log(f"case {w.name}")
    inp, run, pools, inv = _setup(w)
    mass = _check(w, inp, run, inp.q, w.tokens, pools, inv, w.capacity)
    log(f"{w.name}: mass sums {mass.sum(1)}")


def test_token_mass_skvq():
    """The mass does not depend on the channel order; checked with stored
    orders and clipped ranges."""
    w = synth.W_SKVQ.shrink(name="mass_skvq", batch=2, kv_heads=2, q_heads=8, tokens=1999)
    log(f"case {w.name}")
    inp, run, pools, inv = _setup(w)
    _check(w, inp, run, inp.q, w.tokens, pools, inv, w.capacity)


def test_token_mass_after_appends():
    """Appended tokens get their mass at their token index."""
    w = synth.W_APPEND.shrink(name="mass_append", batch=2, kv_heads=2, q_heads=8, tokens=300, append_steps=5)
    log(f"case {w.name}")
    inp, run, pools, inv = _setup(w)
    med = [O.RunningMedian(inp.scores[b]) for b in range(w.batch)]
    for i, st in enumerate(inp.steps):
        run.append(st)
        for b in range(w.batch):
            tier = med[b].decide_and_insert(st["score_new"][b])
            inv[b][tier].append(w.tokens + i)
            for h in range(w.kv_heads):
                pools[(b, h)][tier].add_rows(st["k_new"][b, h][None], st["v_new"][b, h][None])
    n = w.tokens + len(inp.steps)
    _check(w, inp, run, inp.steps[-1]["q"], n, pools, inv, w.capacity)
