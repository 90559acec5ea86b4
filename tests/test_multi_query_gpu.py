"""GPU parity of attention by a block of new query tokens over the packed
tiered cache (kvq_decode_attn_multi): every output row against the oracle's
fp64 attention over the dequantized cache, and every row's log-sum-exp.

Tolerances: outputs 2e-3 (max over rows of max|o - r| / max|r|), as for one
query.  Log-sum-exp: 1e-4 absolute in natural-log units, i.e. 1e-4 relative
in the sum of exponentials; the kernel's scores carry the fp32 rounding of
a dot product and of the scale (a few 1e-7 relative on scores of order 10)
and the sum is fp32, so 1e-4 leaves a margin of about 30 over what is
observed while a wrong scale, base or dropped chunk is off by far more."""
import numpy as np
import pytest

from mixed_precision_kv_amd import kvq, synth
from oracle import kvq_oracle as O
from gpu_harness import GpuRun, TOL, log, oracle_tiers, oracle_unit, to_dev

pytestmark = pytest.mark.gpu

LSE_TOL = 1e-4


def _run_multi(run, qm, max_len=None, with_lse=True):
    import torch
    w = run.w
    M = qm.shape[1]
    ml = max_len or w.tokens
    ws = torch.empty(kvq.multi_workspace_bytes(run.lay, M, w.capacity), dtype=torch.uint8,
                     device=run.cache.device)
    q = to_dev(qm)
    out = torch.empty_like(q)
    lse = torch.full((w.batch, M, w.q_heads), float("nan"), dtype=torch.float32,
                     device=run.cache.device) if with_lse else None
    kvq.decode_attn_multi(run.lay, run.cache, q, M, float(run.scale), ml, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if with_lse else None)


def _check_multi(w, inp, run, qm, units=None):
    out, lse = _run_multi(run, qm)
    _, _, _, inv = oracle_tiers(w, inp)
    g = w.q_heads // w.kv_heads
    M = qm.shape[1]
    errs, lerrs = [], []
    for b in range(w.batch):
        for h in range(w.kv_heads):
            u = b * w.kv_heads + h
            if units is not None and u not in units:
                continue
            pools = oracle_unit(w, inp, inv, b, h)
            kh = np.concatenate([pools[0].k_hat(), pools[1].k_hat()])
            vh = np.concatenate([pools[0].v_hat(), pools[1].v_hat()])
            rows = qm[b, :, h * g:(h + 1) * g].reshape(M * g, -1).astype(np.float64)
            ref, rlse = O.attention_lse_fp64(rows, kh, vh, float(run.scale))
            got = out[b, :, h * g:(h + 1) * g].reshape(M * g, -1)
            errs.append(O.row_rel_err(got, ref))
            lerrs.append(float(np.abs(lse[b, :, h * g:(h + 1) * g].reshape(-1) - rlse).max()))
    log(f"{w.name} M{M}: max row rel err {max(errs):.3e}, max lse err {max(lerrs):.3e}")
    assert max(errs) <= TOL
    assert max(lerrs) <= LSE_TOL


@pytest.mark.parametrize("M", [1, 3, 4, 9])
def test_multi_query_c2_shape(M):
    w = synth.W_LLAMA.shrink(name="c2_small_mq", batch=2, kv_heads=2, q_heads=8, tokens=1999)
    log(f"case {w.name} M{M}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _check_multi(w, inp, run, synth.make_queries(w, M))


@pytest.mark.parametrize("M", [4096, 4093])
def test_multi_query_most_queries(M):
    """The largest block of query tokens the entry point takes (4096, 1024
    query groups of four) and a ragged last group, over a short two-sequence
    cache: every row's output and log-sum-exp."""
    w = synth.W_LLAMA.shrink(name="c2_tiny_mq", batch=2, kv_heads=1, q_heads=4, tokens=613)
    log(f"case {w.name} M{M}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _check_multi(w, inp, run, synth.make_queries(w, M))


@pytest.mark.parametrize("M", [1, 6])
def test_multi_query_skvq(M):
    """Queries gathered through the stored key order, outputs written back
    through the value order."""
    w = synth.W_SKVQ.shrink(name="skvq_small_mq", batch=2, kv_heads=2, q_heads=8, tokens=1999)
    log(f"case {w.name} M{M}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _check_multi(w, inp, run, synth.make_queries(w, M))


@pytest.mark.parametrize("lh,ll,g,T", [(8, 6, 64, 3001), (4, 3, 128, 1201), (8, 7, 32, 777),
                                       (7, 5, 64, 1500), (5, 3, 32, 900), (6, 5, 128, 1400),
                                       (8, 4, 32, 700), (7, 3, 128, 900), (4, 3, 64, 800)])
def test_multi_query_level_pairs(lh, ll, g, T):
    """Every grid 3..8 (table and power-of-two digit paths) and group size."""
    w = synth.W_LLAMA.shrink(name=f"mq_levels_{lh}_{ll}_g{g}", batch=1, kv_heads=2, q_heads=8, tokens=T,
                    levels_hi=lh, levels_lo=ll, group=g)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _check_multi(w, inp, run, synth.make_queries(w, 6))


@pytest.mark.parametrize("T,n_hi", [(1, 0), (17, 17), (193, 96)])
def test_multi_query_edge_sizes(T, n_hi):
    """One token, an empty pool, ragged tails."""
    w = synth.W_LLAMA.shrink(name=f"mq_edge_T{T}_n{n_hi}", batch=2, kv_heads=1, q_heads=4, tokens=T,
                    frac_hi=n_hi / T)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    _check_multi(w, inp, run, synth.make_queries(w, 5))


def test_multi_query_matches_single_query_and_no_lse():
    """Query 0 of a block equals kvq_decode_attn on that query (both within the
    oracle bound), and a null lse pointer is accepted."""
    w = synth.W_LLAMA.shrink(name="mq_vs_one", batch=2, kv_heads=2, q_heads=8, tokens=1500)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    qm = synth.make_queries(w, 4)
    out, _ = _run_multi(run, qm, with_lse=False)
    one = run.decode(np.ascontiguousarray(qm[:, 0]))
    d = np.abs(out[:, 0].astype(np.float64) - one.astype(np.float64)).max()
    den = np.abs(one.astype(np.float64)).max()
    log(f"max |multi - single| / max|single| = {d / den:.3e}")
    assert d / den <= 2 * TOL
