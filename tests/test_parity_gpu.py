"""GPU parity on sizes the oracle finishes in seconds: every output of the HIP
path against the oracle, element by element (bit-exact for ranks, token
maps, counters, codes, words and fp16 scale/zero; attention within 2e-3)."""
import numpy as np
import pytest

from mixed_precision_kv_amd import synth
from oracle import kvq_oracle as O
import layout_view as LV
from gpu_harness import (GpuRun, TOL, check_kchan as _check_kchan, check_tiered as _check_tiered,
                         compare_tiered_unit, log, oracle_tiers, oracle_unit, oracle_unit_attention)

pytestmark = pytest.mark.gpu



SMALL = [
    synth.W_SINGLE,                                                            # config 1 at full size
    synth.W_LLAMA.shrink(name="c2_small", batch=2, kv_heads=2, q_heads=8, tokens=1999),
    synth.W_LONG.shrink(name="c3_small", batch=1, kv_heads=2, q_heads=8, tokens=3001),
    synth.W_APPEND.shrink(name="c4_prefix_small", batch=3, kv_heads=2, q_heads=8, tokens=777, append_steps=0),
    synth.W_SKVQ.shrink(name="skvq_small", batch=2, kv_heads=2, q_heads=8, tokens=1999),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_tiered_quantize_and_decode(w):
    log(f"case {w.name} B{w.batch} H{w.kv_heads} T{w.tokens}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


@pytest.mark.parametrize("lh,ll,g", [(4, 3, 128), (7, 6, 64), (8, 7, 32), (5, 4, 64)])
def test_tiered_level_pairs(lh, ll, g):
    """Every grid size 3..8 and group size of the tiered path (codes per
    word 20, 16, 13, 12, 11, 10), with decode over the result."""
    w = synth.W_LLAMA.shrink(name=f"levels_{lh}_{ll}_g{g}", batch=2, kv_heads=2, q_heads=8, tokens=1201,
                    levels_hi=lh, levels_lo=ll, group=g)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


@pytest.mark.parametrize("lh,ll,g,clip,reorder,T", [
    (6, 5, 32, 0.9, True, 1201),
    (8, 6, 64, 0.5, True, 3001),
    (4, 3, 128, 0.75, True, 777),
    (7, 6, 32, 0.8, False, 1201),      # clipping alone (natural channel order)
    (5, 4, 64, 0.0, True, 1201),       # stored orders alone
    (8, 7, 32, 1.0, True, 17),         # clip factor 1 with orders, one ragged tile
    (3, 3, 32, 0.3, True, 640),
])
def test_skvq_variants(lh, ll, g, clip, reorder, T):
    """Stored channel orders and clipped group ranges (SKVQ, Abstract) over
    grid sizes 3..8 and groups of 32, 64 and 128: codes, words and fp16
    (scale, zero) bit-exact in stored order, decode in channel order."""
    w = synth.W_SKVQ.shrink(name=f"skvq_{lh}_{ll}_g{g}_c{clip}_r{int(reorder)}_T{T}", batch=2, kv_heads=2,
                            q_heads=8, tokens=T, levels_hi=lh, levels_lo=ll, group=g, clip=clip,
                            reorder=reorder)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


def test_skvq_degenerate_groups():
    """Clipping and stored orders on constant groups (scale 0), signed
    zeros, ranges that clip to one fp16 value, and tiny ranges whose
    clipped fp16 scale is subnormal."""
    w = synth.W_SKVQ.shrink(name="skvq_degenerate", batch=2, kv_heads=2, q_heads=8, tokens=500, clip=0.5)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    inp.k[0, 10:20, 0, :] = np.float16(0.75)                 # constant rows
    inp.v[1, 5:9, 1, :] = np.float16(-2.0)
    inp.k[1, 30, 1, :] = np.float16(-0.0)
    inp.v[0, 40, 0, ::2] = np.float16(-0.0)
    inp.v[0, 40, 0, 1::2] = np.float16(0.0)
    tiny = np.float16(2.0 ** -24)
    inp.k[0, 50:60, 1, :] = (np.arange(128) % 8).astype(np.float16) * tiny
    inp.v[1, 61:70, 0, :] = (np.arange(128) % 3).astype(np.float16) * tiny   # clipped range: one value
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


@pytest.mark.parametrize("T,n_hi", [(1, 0), (1, 1), (17, 0), (17, 17), (193, 96), (640, 320)])
def test_tiered_edge_sizes(T, n_hi):
    w = synth.W_LLAMA.shrink(name=f"edge_T{T}_n{n_hi}", batch=2, kv_heads=1, q_heads=4, tokens=T,
                    frac_hi=n_hi / T)
    assert w.n_hi == n_hi
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


@pytest.mark.parametrize("T", [32769, 70001])
def test_tiered_long_sequences_with_ties(T):
    """Sequences longer than one workgroup's LDS of sorted keys (the ranks
    add partial counts over groups of blocks, the last group partial), with
    runs of equal scores across block and group boundaries."""
    w = synth.W_LONG.shrink(name=f"long_T{T}", batch=2, kv_heads=1, q_heads=4, tokens=T)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    inp.scores[0] = np.round(inp.scores[0] * 4) / 4            # few distinct values: long tie runs
    inp.scores[1, 30000:36000] = np.float32(1.0)                # one run over the group boundary
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


def test_tiered_longest_sequence():
    """The longest sequence the rank kernels take (262144 tokens: eight
    groups of eight 4096-token blocks), with long runs of equal scores, at
    the long-context workload's 8/6 levels and 64-channel groups; every
    rank, slot, word and scale, and the attention, against the oracle."""
    w = synth.W_LONG.shrink(name="longest_T262144", batch=1, kv_heads=1, q_heads=4, tokens=262144)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    inp.scores[0, ::3] = np.round(inp.scores[0, ::3] * 8) / 8   # tie runs in every block and group
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


def test_tiered_many_short_units():
    """More (sequence, KV head) units than workgroups resident on the chip
    (256 x 8 = 2048 units of 45 tokens: one chunk per unit, several rounds
    of workgroups, a one-partial merge), ragged tiers (22 / 23 slots)."""
    w = synth.W_LLAMA.shrink(name="many_units_T45", batch=256, kv_heads=8, q_heads=32, tokens=45)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


def test_tiered_ties_zeros_and_constant_groups():
    """Equal scores (stable order decides), -0/+0 scores, constant groups
    (scale 0), signed zeros in the data."""
    w = synth.W_LLAMA.shrink(name="degenerate", batch=2, kv_heads=2, q_heads=8, tokens=500)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    inp.scores[0, :] = np.float32(1.5)                       # all equal
    inp.scores[1, ::3] = np.float32(0.0)
    inp.scores[1, 1::7] = np.float32(-0.0)
    inp.k[0, 10:20, 0, :] = np.float16(0.75)                 # constant rows -> s = 0
    inp.v[1, 5:9, 1, 32:64] = np.float16(-2.0)
    inp.k[1, 30, 1, :8] = np.float16(-0.0)
    inp.v[0, 40, 0, 3] = np.float16(-0.0)
    inp.v[0, 40, 0, 4] = np.float16(0.0)
    # tiny ranges: subnormal fp16 scales far below range / (L - 1), so the
    # quotient exceeds the top level and the code must be clamped
    tiny = np.float16(2.0 ** -24)
    inp.k[0, 50:60, 1, :32] = (np.arange(32) % 8).astype(np.float16) * tiny
    inp.v[1, 61:70, 0, 64:96] = (np.arange(32) % 7).astype(np.float16) * tiny - np.float16(3e-7)
    inp.k[1, 71:80, 0, 96:128] = np.linspace(-4e-7, 5e-7, 32).astype(np.float16)
    run = GpuRun(w, inp)
    run.quantize()
    _check_tiered(w, inp, run)


@pytest.mark.parametrize("T", [100, 255, 256, 434, 1408, 2000])
def test_kchan_quantize_and_decode(T):
    w = synth.W_KCHAN.shrink(name=f"c5_T{T}", batch=2, kv_heads=2, q_heads=8, tokens=T)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_kchan(w, inp, run)


@pytest.mark.parametrize("kl,vl,vg,spv,win,T", [
    (3, 4, 64, 1, 64, 1000),      # VALU decode, one sparse entry, short window
    (8, 6, 128, 0, 0, 777),       # no sparse entries, no window beyond the ragged block tail
    (16, 8, 32, 5, 200, 1500),    # 16-level keys (generic key kernel), five sparse entries
    (4, 3, 32, 2, 17, 300),       # the matrix-core shape with an odd window
    (9, 16, 64, 3, 128, 900),     # values past 8 levels (generic pool quantizer)
])
def test_kchan_other_shapes(kl, vl, vg, spv, win, T):
    """Per-channel-key caches outside the matrix-core kernel's shape: the
    generic key quantizer and the VALU decode (quantized chunks and fp16
    window chunks)."""
    w = synth.W_KCHAN.shrink(name=f"kchan_k{kl}_v{vl}_g{vg}_s{spv}_w{win}_T{T}", batch=2, kv_heads=2, q_heads=8,
                    tokens=T, k_levels=kl, v_levels=vl, v_group=vg, sparse_per_vec=spv, window=win)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    _check_kchan(w, inp, run)


def test_kchan_outlier_ties_and_degenerate_blocks():
    """Sparse outliers under magnitude ties (lower channel wins, +x and -x
    tie), all-zero and -0 key rows (channels 0 and 1 are taken), constant
    channels (scale 0) and tiny channel ranges (subnormal scales)."""
    w = synth.W_KCHAN.shrink(name="c5_edges", batch=1, kv_heads=2, q_heads=8, tokens=640)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    k = inp.k
    k[0, 3, 0, :] = np.float16(0.0)                          # all zero
    k[0, 4, 0, :] = np.float16(-0.0)                         # all -0
    k[0, 5, 0, 40] = np.float16(7.0)                         # three-way tie for the top
    k[0, 5, 0, 20] = np.float16(-7.0)
    k[0, 5, 0, 90] = np.float16(7.0)
    k[0, 6, 1, :] = np.float16(1.5)                          # every magnitude equal
    k[0, 128:256, 1, 17] = np.float16(0.25)                  # constant channel in a block
    k[0, 256:384, 0, 33] = (np.arange(128) % 8).astype(np.float16) * np.float16(2.0 ** -24)
    k[0, 384:512, 1, 64] = np.float16(-0.0)
    run = GpuRun(w, inp)
    run.quantize()
    _check_kchan(w, inp, run)


@pytest.mark.parametrize("w", [
    synth.W_APPEND.shrink(name="c4_small", batch=3, kv_heads=2, q_heads=8, tokens=300, append_steps=40),
    synth.W_SKVQ.shrink(name="skvq_append_small", batch=3, kv_heads=2, q_heads=8, tokens=300, append_steps=40),
], ids=lambda w: w.name)
def test_append_then_decode_small(w):
    """Generation-time quantization: every step's tier decision, slot, words
    and the attention after it, against the running-median oracle (also with
    stored channel orders and clipped ranges)."""
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    rank, tokmap, counts, inv = oracle_tiers(w, inp)
    med = [O.RunningMedian(inp.scores[b]) for b in range(w.batch)]
    pools = {(b, h): oracle_unit(w, inp, inv, b, h)
             for b in range(w.batch) for h in range(w.kv_heads)}
    tok = [list(tokmap[b]) for b in range(w.batch)]
    for i, st in enumerate(inp.steps):
        run.append(st)
        for b in range(w.batch):
            tier = med[b].decide_and_insert(st["score_new"][b])
            slot = pools[(b, 0)][tier].n
            tok[b].append(slot | (tier << 31))
            for h in range(w.kv_heads):
                pools[(b, h)][tier].add_rows(st["k_new"][b, h][None], st["v_new"][b, h][None])
        buf = run.buf()
        n = w.tokens + i + 1
        assert np.array_equal(LV.tokmap(buf, run.lay)[:, :n], np.array(tok, dtype=np.uint32)), f"step {i}"
        cnt = LV.counters(buf, run.lay)
        assert np.all(cnt[:, 0] == n) and np.all(cnt[:, 3] == 0)
        assert np.array_equal(LV.sorted_scores(buf, run.lay)[:, :n],
                              np.array([m.s for m in med], dtype=np.float32)), f"sorted step {i}"
        out = run.decode(st["q"], max_len=n)
        errs = []
        for b in range(w.batch):
            for h in range(w.kv_heads):
                p = pools[(b, h)]
                kh = np.concatenate([p[0].k_hat(), p[1].k_hat()])
                vh = np.concatenate([p[0].v_hat(), p[1].v_hat()])
                ref = oracle_unit_attention(w, st["q"], b, h, kh, vh, run.scale)
                errs.append(O.row_rel_err(out[b, h * 4:(h + 1) * 4], ref))
        assert max(errs) <= TOL, f"step {i}: {max(errs)}"
    buf = run.buf()
    for (b, h), p in pools.items():
        compare_tiered_unit(buf, run.lay, p, b * w.kv_heads + h, f"after appends b{b} h{h}")


def test_append_pool_full_flag():
    """A sequence whose tier pool is full is left unchanged and flagged."""
    w = synth.W_APPEND.shrink(name="c4_full", batch=2, kv_heads=1, q_heads=4, tokens=64, append_steps=2)
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp)
    run.quantize()
    st = dict(inp.steps[0])
    st["score_new"] = np.array([1e30, -1e30], dtype=np.float32)   # b0 -> hi, b1 -> lo
    run.append(st)
    run.append(st)
    before = LV.counters(run.buf(), run.lay).copy()
    assert before[:, 0].tolist() == [66, 66] and before[:, 3].tolist() == [0, 0]
    run.append(st)                                                  # pools hold 32 + 2 slots
    after = LV.counters(run.buf(), run.lay)
    assert after[:, 3].tolist() == [1, 1]
    assert np.array_equal(after[:, :3], before[:, :3])


def test_stream_read_probe_reads_every_word_once():
    """The bandwidth probe's sink: the xor of the per-workgroup words equals
    the xor of every word of the buffer (each word read exactly once)."""
    import torch
    from mixed_precision_kv_amd import kvq
    rng = np.random.default_rng(5)
    words = rng.integers(0, 2**32, size=(1 << 20) + 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    for nwg in (1, 7, 300):
        sink = torch.zeros(nwg, dtype=torch.int32, device="cuda:0")
        kvq.stream_read(buf, sink, nwg)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(words), nwg
