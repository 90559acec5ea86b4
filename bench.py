"""Throughput of the mixed-precision KV-cache hot path on one MI355X.

Default workload: generation over a packed cache (batch 64, 8 KV heads, 32
query heads, head_dim 128; a 16384-token prefix on 6/5-level grids with
groups of 32, then 256 generation steps).  One step is the whole hot path
over that batch: quantize-on-write of the prefix (rank, tier split, group
quantize, base-L packing of K and V), then 256 times: append one token per
sequence (running-median tier, quantize, pack) and one decode-attention step
of every sequence over the packed cache (split over the context, merged by
log-sum-exp).  Inputs, including every step's new tokens and queries, are
synthetic and resident in HBM before the timed region.

Prints one JSON line.  `value` is decode-attention context tokens per second
per query head over the whole step: the sum over the 256 decodes of
B * Hq * (tokens in the cache) divided by the step time (prefix quantize and
appends included).  Every quantize, append and decode of the timed steps is
also bracketed by HIP events on the stream it runs on; `decode` and
`quantize` report those live durations and `roofline` the dominant entry
point (decode) against 8 TB/s with its algorithmic bytes.  Workloads
without generation steps (--config) time quantize + one decode per step and
rotate cache replicas so that decode reads come from HBM rather than the
256 MB Infinity Cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0      # dense fp16 matrix-core peak
DECODE_SOURCES = ("decode.hip", "decode_mfma.hip", "mfma_util.h", "unpack.h", "digits.h", "tiling.h",
                  "common.h", "internal.h")
QUANTIZE_SOURCES = ("quantize.hip", "rank.hip", "digits.h", "tiling.h", "common.h", "internal.h")


def packed_decode_bytes(lay, counts):
    """Algorithmic bytes one decode reads: every packed word and (scale, zero)
    pair of every stored token, the query and the output."""
    c = lay.cfg
    D = c.head_dim
    total = 0
    if c.mode == 0:
        ng = D // c.group
        for b in range(c.batch):
            for p in range(2):
                n = int(counts[b][p])
                per_unit = n * lay.kw[p] * 4 + 2 * n * ng * 4 + -(-n // lay.nv[p]) * D * 4
                total += per_unit * c.kv_heads
    else:
        raise NotImplementedError
    total += 2 * c.batch * c.q_heads * D * 2
    return total


def kchan_decode_bytes(lay, T):
    """Algorithmic bytes one per-channel-key decode reads: key words, key
    (scale, zero) per (channel, block), sparse entries, value words and
    (scale, zero), the fp16 window, the query and the output."""
    c = lay.cfg
    D, U = c.head_dim, c.batch * c.kv_heads
    n_q = c.k_block * ((T - c.window) // c.k_block)
    per_unit = (n_q * lay.kw[0] * 4 + (n_q // c.k_block) * D * 4 + n_q * c.sparse_per_vec * 4
                + -(-n_q // lay.vnv) * D * 4 + n_q * (D // c.v_group) * 4 + (T - n_q) * D * 2 * 2)
    return U * per_unit + 2 * c.batch * c.q_heads * D * 2


def quantize_bytes(w, lay):
    """Algorithmic bytes of quantize: fp16 K and V and the scores read once;
    packed cache, token map, sorted scores and ranks written once."""
    B, T, H, D = w.batch, w.tokens, w.kv_heads, w.head_dim
    rd = 2 * B * T * H * D * 2 + B * T * 4
    counts = [[w.n_hi, T - w.n_hi]] * B
    wr = packed_decode_bytes(lay, counts) - 2 * B * w.q_heads * D * 2 + 3 * B * T * 4
    return rd + wr


def kernel_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixed_precision_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, khash, workload):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, only if the
    kernel source is unchanged since the counters were taken and they were
    taken on this workload."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    e = tr.get(kernel)
    if not e or e.get("source_hash") != khash or e.get("workload") != workload:
        return None
    return e.get("bytes_per_launch")


# ----------------------------------------------------------- cpu baseline ---
def cpu_share():
    """CPUs this process may use: its affinity set, bounded by a cgroup CPU
    quota and by OMP_NUM_THREADS when the environment sets one (a GPU host
    may allot a share of its cores to each GPU)."""
    n = len(os.sched_getaffinity(0))
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, math.ceil(int(quota) / int(period))))
    except (OSError, ValueError):
        pass
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _one_blas_thread():
    try:
        import threadpoolctl
        threadpoolctl.threadpool_limits(1)
    except ImportError:
        pass


def _oracle_unit(args):
    """Oracle work of one (sequence, KV head): quantize + pack of its prefix,
    then `gen` generation steps (running-median tier, quantize + store of the
    new token, fp64 attention over the whole cache), or one fp64 decode when
    the workload has no generation steps.  Returns (prefix s, per-step s)."""
    import numpy as np
    from oracle import kvq_oracle as O
    k_unit, v_unit, inv_b, scores_b, q_group, w_fields, scale, gen = args
    L_hi, L_lo, G, skvq = w_fields
    t0 = time.perf_counter()
    pools = O.quantize_tiered_unit(k_unit, v_unit, inv_b, L_hi, L_lo, G, **skvq)
    for p in pools:
        p.k_words(), p.v_words()
    t1 = time.perf_counter()
    if not gen:
        kh = np.concatenate([pools[0].k_hat(), pools[1].k_hat()])
        vh = np.concatenate([pools[0].v_hat(), pools[1].v_hat()])
        O.decode_unit(q_group, kh, vh, scale)
        return t1 - t0, time.perf_counter() - t1
    med = O.RunningMedian(scores_b)
    for st in gen:
        tier = med.decide_and_insert(st["score"])
        pools[tier].add_rows(st["k"][None], st["v"][None])
        pools[tier].k_words(), pools[tier].v_words()
        kh = np.concatenate([pools[0].k_hat(), pools[1].k_hat()])
        vh = np.concatenate([pools[0].v_hat(), pools[1].v_hat()])
        O.decode_unit(st["q"], kh, vh, scale)
    return t1 - t0, (time.perf_counter() - t1) / len(gen)


def cpu_baseline(w, inp, scale, units_per_worker, gen_sample, workers):
    """The oracle as it is, on the host's CPU share: rank + tier split of
    every sequence, then for a sample of (sequence, KV head) units (spread
    over `workers` processes) the quantize + pack of the prefix and, for a
    generation workload, `gen_sample` of its append + fp64 decode steps.
    The measured per-unit times are scaled to one whole bench step (every
    unit, every generation step) at `workers`-way parallelism."""
    import numpy as np
    from mixed_precision_kv_amd import synth
    from oracle import kvq_oracle as O
    t0 = time.perf_counter()
    rank = O.rank_desc(inp.scores)
    _, _, inv = O.tiers_and_slots(rank, w.n_hi)
    t_rank = time.perf_counter() - t0
    g = w.q_heads // w.kv_heads
    n_all = w.batch * w.kv_heads
    n_units = min(n_all, units_per_worker * workers)
    stride = max(1, n_all // n_units)
    units = [(u // w.kv_heads, u % w.kv_heads) for u in range(0, n_all, stride)][:n_units]
    orders = synth.channel_orders(w) if w.reorder else None

    def skvq(h):
        kw = dict(order_k=orders[0, h], order_v=orders[1, h]) if w.reorder else {}
        return dict(kw, clip=w.clip) if w.clip else kw

    n_gen = min(gen_sample, len(inp.steps))

    def gen_of(b, h):
        return [dict(score=float(st["score_new"][b]), k=st["k_new"][b, h], v=st["v_new"][b, h],
                     q=st["q"][b, h * g:(h + 1) * g].astype(np.float64)) for st in inp.steps[:n_gen]]

    jobs = [(np.ascontiguousarray(inp.k[b, :, h]), np.ascontiguousarray(inp.v[b, :, h]), inv[b],
             inp.scores[b], inp.q[b, h * g:(h + 1) * g].astype(np.float64),
             (w.levels_hi, w.levels_lo, w.group, skvq(h)), scale, gen_of(b, h)) for b, h in units]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers, initializer=_one_blas_thread) as pool:
        res = pool.map(_oracle_unit, jobs, chunksize=1)
    t_units = time.perf_counter() - t0
    t_pre = float(np.mean([r[0] for r in res]))
    t_gen = float(np.mean([r[1] for r in res]))
    steps = w.append_steps if w.append_steps else 1
    cpu_s = n_all * (t_pre + steps * t_gen)          # CPU-seconds of one whole step
    t_step = t_rank + cpu_s / workers
    if w.append_steps:
        ctx = w.batch * w.q_heads * sum(w.tokens + i + 1 for i in range(w.append_steps))
        sample = (f"rank+tiers of all {w.batch} sequences; for {len(units)} of {n_all} (sequence, KV head) "
                  f"units: prefix quantize+pack and {n_gen} of {w.append_steps} generation steps "
                  f"(running-median append, fp64 attention over the cache); per-unit times scaled to "
                  f"every unit and every step at {workers}-way parallelism")
    else:
        ctx = w.batch * w.q_heads * w.tokens
        sample = (f"rank+tiers of all {w.batch} sequences; quantize+pack+fp64 attention of {len(units)} of "
                  f"{n_all} (sequence, KV head) units, scaled to the batch at {workers}-way parallelism")
    return dict(value=ctx / t_step, unit="decode-attention context tokens/s per query head",
                cores=workers, kind="oracle", sample=sample, host_cpus=os.cpu_count(),
                cpu_model=cpu_model(), seconds=round(t_rank + t_units, 3),
                est_step_s=round(t_step, 3))


# ------------------------------------------------------------------- main ---
def _timed(torch, stream, fn, iters):
    """Median and spread (ms) of fn(i) over iters calls, HIP events on `stream`."""
    import numpy as np
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i in range(iters):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def stream_read_gbs(torch, kvq, dev, stream, nbytes=1 << 30, iters=10):
    """Achievable HBM read rate: the library's read-stream probe over a buffer
    four times the 256 MB infinity cache, median of `iters` launches."""
    import numpy as np
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    nwg = 4096
    sink = torch.zeros(nwg, dtype=torch.int32, device=dev)
    for _ in range(3):
        kvq.stream_read(buf, sink, nwg, stream=stream)
    ms = _timed(torch, stream, lambda i: kvq.stream_read(buf, sink, nwg, stream=stream), iters)[0]
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def sweep_one(w, args, torch, np, kvq, synth, dev):
    """Quantize and decode (and, for the append workload, append + decode per
    generation step) of one workload, inputs resident in HBM."""
    print(f"[sweep] {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)
    lay = kvq.layout_init(kvq.config_for(w))
    stream = torch.cuda.current_stream()
    k = torch.from_numpy(inp.k).to(dev)
    v = torch.from_numpy(inp.v).to(dev)
    scores = None if inp.scores is None else torch.from_numpy(inp.scores).to(dev)
    q = torch.from_numpy(inp.q).to(dev)
    out = torch.empty_like(q)
    max_len = w.tokens + w.append_steps
    wsq = torch.empty(max(1, kvq.workspace_bytes(lay, kvq.OP_QUANTIZE, w.tokens)), dtype=torch.uint8, device=dev)
    wsd = torch.empty(max(1, kvq.workspace_bytes(lay, kvq.OP_DECODE, max_len)), dtype=torch.uint8, device=dev)
    R = 1 if w.append_steps else max(1, math.ceil(1.0e9 / lay.total_bytes))
    caches = [torch.zeros(lay.total_bytes, dtype=torch.uint8, device=dev) for _ in range(R)]
    if w.reorder:
        for c in caches:
            kvq.set_channel_order(lay, c, synth.channel_orders(w), stream=stream)
    scale = 1.0 / math.sqrt(w.head_dim)
    tiered = w.mode == synth.TIERED

    def quantize(i):
        kvq.quantize(lay, caches[i % R], k, v, scores, w.tokens, w.n_hi if tiered else 0, None, wsq,
                     stream=stream)

    def decode(i, c=None):
        kvq.decode_attn(lay, caches[i % R] if c is None else c, q, scale, max_len, out, wsd, stream=stream)

    for i in range(R):
        quantize(i)
    torch.cuda.synchronize()
    q_ms = _timed(torch, stream, quantize, 10)
    rd = 2 * w.batch * w.tokens * w.kv_heads * w.head_dim * 2
    if tiered:
        counts = [[w.n_hi, w.tokens - w.n_hi]] * w.batch
        dec_bytes = packed_decode_bytes(lay, counts)
        q_bytes = quantize_bytes(w, lay)
    else:
        dec_bytes = kchan_decode_bytes(lay, w.tokens)
        q_bytes = rd + dec_bytes - 2 * w.batch * w.q_heads * w.head_dim * 2
    for i in range(R):
        quantize(i)
    for i in range(3):
        decode(i)
    d_ms = _timed(torch, stream, decode, 30)
    res = {"workload": w.name, "config": {"batch": w.batch, "kv_heads": w.kv_heads, "q_heads": w.q_heads,
                                           "context": w.tokens, "mode": w.mode},
           "quantize": {"ms": q_ms[0], "ms_p10": q_ms[1], "ms_p90": q_ms[2], "bytes": q_bytes,
                        "gbs": round(q_bytes / (q_ms[0] * 1e-3) / 1e9, 1),
                        "frac_hbm": round(q_bytes / (q_ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "decode": {"ms": d_ms[0], "ms_p10": d_ms[1], "ms_p90": d_ms[2], "bytes": dec_bytes,
                      "gbs": round(dec_bytes / (d_ms[0] * 1e-3) / 1e9, 1),
                      "frac_hbm": round(dec_bytes / (d_ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "ctx_tokens_per_s_per_qhead": w.batch * w.q_heads * w.tokens / (d_ms[0] * 1e-3),
                      "replicas": R}}
    if tiered:
        # decode that also reports every token's attention mass
        mass = torch.empty((w.batch, max_len), dtype=torch.float32, device=dev)
        wsm = torch.empty(kvq.workspace_bytes(lay, kvq.OP_DECODE_MASS, max_len), dtype=torch.uint8, device=dev)

        def decode_mass(i):
            kvq.decode_attn_mass(lay, caches[i % R], q, scale, max_len, out, mass, wsm, stream=stream)

        for i in range(3):
            decode_mass(i)
        dm_ms = _timed(torch, stream, decode_mass, 30)
        res["decode_mass"] = {"ms": dm_ms[0], "ms_p10": dm_ms[1], "ms_p90": dm_ms[2],
                              "overhead_vs_decode": round(dm_ms[0] / d_ms[0] - 1.0, 4)}
    if tiered and args.multi_queries > 0 and not w.rope_theta:
        # a block of M new query tokens per sequence over the same caches
        M = args.multi_queries
        qm = torch.from_numpy(synth.make_queries(w, M)).to(dev)
        om = torch.empty_like(qm)
        lse = torch.empty((w.batch, M, w.q_heads), dtype=torch.float32, device=dev)
        wsm = torch.empty(max(1, kvq.multi_workspace_bytes(lay, M, max_len)), dtype=torch.uint8, device=dev)

        def multi(i):
            kvq.decode_attn_multi(lay, caches[i % R], qm, M, scale, max_len, om, lse, wsm, stream=stream)

        for i in range(3):
            multi(i)
        m_ms = _timed(torch, stream, multi, 20)
        m_bytes = dec_bytes + 2 * w.batch * M * w.q_heads * w.head_dim * 2 - 2 * w.batch * w.q_heads * w.head_dim * 2
        m_flop = 2048.0 * M * w.batch * w.kv_heads * w.tokens
        res["multi_query"] = {"queries": M, "ms": m_ms[0], "ms_p10": m_ms[1], "ms_p90": m_ms[2],
                              "bytes": m_bytes, "gbs": round(m_bytes / (m_ms[0] * 1e-3) / 1e9, 1),
                              "frac_hbm": round(m_bytes / (m_ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "tflops": round(m_flop / (m_ms[0] * 1e-3) / 1e12, 2),
                              "frac_fp16_mfma": round(m_flop / (m_ms[0] * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                              "ctx_tokens_per_s_per_qhead": M * w.batch * w.q_heads * w.tokens / (m_ms[0] * 1e-3)}
    if w.append_steps:
        # generation: each step appends one token per sequence, then decodes
        quantize(0)
        torch.cuda.synchronize()
        steps = [dict(k=torch.from_numpy(st["k_new"]).to(dev), v=torch.from_numpy(st["v_new"]).to(dev),
                      s=torch.from_numpy(st["score_new"]).to(dev), q=torch.from_numpy(st["q"]).to(dev))
                 for st in inp.steps]
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in steps]
        for i, st in enumerate(steps):
            ev[i][0].record(stream)
            kvq.append(lay, caches[0], st["k"], st["v"], st["s"], stream=stream)
            ev[i][1].record(stream)
            kvq.decode_attn(lay, caches[0], st["q"], scale, max_len, out, wsd, stream=stream)
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        a_t = np.array([e[0].elapsed_time(e[1]) for e in ev])
        dd_t = np.array([e[1].elapsed_time(e[2]) for e in ev])
        raw = caches[0][lay.counters:lay.counters + w.batch * 16].cpu().numpy().tobytes()
        cnt = np.frombuffer(raw, dtype=np.int32).reshape(w.batch, 4)
        end_counts = [[int(cnt[b, 1]), int(cnt[b, 2])] for b in range(w.batch)]
        start_bytes = dec_bytes
        end_bytes = packed_decode_bytes(lay, end_counts)
        mid_bytes = 0.5 * (start_bytes + end_bytes)
        res["append"] = {"steps": len(steps), "append_ms": float(np.median(a_t)),
                         "decode_ms": float(np.median(dd_t)),
                         "step_ms": float(np.median(a_t + dd_t)),
                         "decode_gbs": round(mid_bytes / (float(np.median(dd_t)) * 1e-3) / 1e9, 1),
                         "decode_frac_hbm": round(mid_bytes / (float(np.median(dd_t)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "final_length": int(cnt[0, 0])}
    print(f"[sweep] {w.name}: quantize {q_ms[0] * 1e3:.1f} us, decode {d_ms[0] * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    del caches, k, v
    torch.cuda.empty_cache()
    return res


def gen_step_counts(torch, kvq, lay, cache, quantize, steps, w, stream):
    """Tier counts of every sequence after each generation step (one untimed
    pass that reads the counters back after every append; the timed steps
    replay the same inputs, so they see the same counts)."""
    import numpy as np
    quantize()
    counts = []
    for st in steps:
        kvq.append(lay, cache, st["k"], st["v"], st["s"], stream=stream)
        raw = cache[lay.counters:lay.counters + w.batch * 16].cpu().numpy().tobytes()
        cnt = np.frombuffer(raw, dtype=np.int32).reshape(w.batch, 4)
        assert not cnt[:, 3].any(), "append flagged a sequence"
        counts.append([[int(cnt[b, 1]), int(cnt[b, 2])] for b in range(w.batch)])
    torch.cuda.synchronize()
    return counts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c4_append_b64_t16k")
    ap.add_argument("--decode-iters", type=int, default=100,
                    help="workloads without generation steps, and --only decode: decode calls timed")
    ap.add_argument("--replicas", type=int, default=0, help="decode cache replicas (0: auto, >= 1 GB)")
    ap.add_argument("--cpu-units-per-worker", type=int, default=4)
    ap.add_argument("--cpu-gen-steps", type=int, default=160,
                    help="generation steps per sampled unit in the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="time quantize / decode (and append) of every workload; one JSON line each")
    ap.add_argument("--sweep-only", default="", help="with --sweep: just these workloads (comma-separated)")
    ap.add_argument("--multi-queries", type=int, default=16,
                    help="with --sweep: also time attention of this many new query tokens per "
                         "sequence over each tiered cache (0: skip)")
    ap.add_argument("--only", choices=["all", "decode", "quantize", "copy"], default="all",
                    help="profiling aid: run just one kernel family (no JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (independent "
              "(sequence, KV head) units would shard across GPUs with no exchange); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    from mixed_precision_kv_amd import synth

    w = None if args.sweep else synth.BY_NAME[args.config]
    if w is not None:
        assert w.mode == "tiered", "the step bench covers the tiered workloads"
        print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)
        inp = synth.make_inputs(w, steps=None if args.only == "all" else 0)
    scale = 1.0 / math.sqrt(128)

    # the oracle baseline runs before anything touches the GPU (its workers are forked)
    cpu = None
    if w is not None and args.only == "all" and not args.no_cpu_baseline:
        workers = cpu_share()
        print(f"[bench] cpu baseline (oracle) on {workers} of {os.cpu_count()} host CPUs", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(w, inp, float(np.float32(scale)), args.cpu_units_per_worker, args.cpu_gen_steps,
                           workers)
        print(f"[bench] cpu baseline done in {cpu['seconds']} s", file=sys.stderr, flush=True)

    import torch
    from mixed_precision_kv_amd import kvq

    dev = torch.device("cuda:0")
    if args.sweep:
        rg = stream_read_gbs(torch, kvq, dev, torch.cuda.current_stream())
        print(json.dumps({"probe": "stream_read", "bytes": 1 << 30, "gbs": round(rg, 1),
                          "frac_hbm": round(rg / HBM_PEAK_GBS, 4)}), flush=True)
        for cw in synth.CONFIGS + [synth.W_SKVQ, synth.W_ROPE, synth.W_ROPE_LONG]:
            if args.sweep_only and cw.name not in args.sweep_only.split(","):
                continue
            print(json.dumps(sweep_one(cw, args, torch, np, kvq, synth, dev)), flush=True)
        return

    lay = kvq.layout_init(kvq.config_for(w))
    stream = torch.cuda.current_stream()
    if args.only == "copy":
        # plain copy of a known size: calibrates the PMC byte counters
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: 5 x {n} bytes", file=sys.stderr)
        return

    k = torch.from_numpy(inp.k).to(dev)
    v = torch.from_numpy(inp.v).to(dev)
    scores = torch.from_numpy(inp.scores).to(dev)
    q = torch.from_numpy(inp.q).to(dev)
    out = torch.empty_like(q)
    ranks = torch.empty((w.batch, w.tokens), dtype=torch.int32, device=dev)
    max_len = w.capacity
    wsq = torch.empty(kvq.workspace_bytes(lay, kvq.OP_QUANTIZE, w.tokens), dtype=torch.uint8, device=dev)
    wsd = torch.empty(kvq.workspace_bytes(lay, kvq.OP_DECODE, max_len), dtype=torch.uint8, device=dev)
    gen = bool(w.append_steps) and args.only == "all"
    R = 1 if w.append_steps else (args.replicas or max(1, math.ceil(1.0e9 / lay.total_bytes)))
    caches = [torch.zeros(lay.total_bytes, dtype=torch.uint8, device=dev) for _ in range(R)]
    if w.reorder:
        for c in caches:
            kvq.set_channel_order(lay, c, synth.channel_orders(w), stream=stream)

    def quantize(i=0):
        kvq.quantize(lay, caches[i % R], k, v, scores, w.tokens, w.n_hi, ranks, wsq, stream=stream)

    def decode(i=0, qq=None):
        kvq.decode_attn(lay, caches[i % R], q if qq is None else qq, scale, max_len, out, wsd, stream=stream)

    for i in range(R):
        quantize(i)
    torch.cuda.synchronize()
    print(f"[bench] {R} cache(s) of {lay.total_bytes / 1e6:.1f} MB ready", file=sys.stderr, flush=True)

    if args.only == "decode":
        for i in range(args.decode_iters):
            decode(i)
        torch.cuda.synchronize()
        return
    if args.only == "quantize":
        for i in range(args.steps):
            quantize(i)
        torch.cuda.synchronize()
        return

    steps = []
    if gen:
        steps = [dict(k=torch.from_numpy(st["k_new"]).to(dev), v=torch.from_numpy(st["v_new"]).to(dev),
                      s=torch.from_numpy(st["score_new"]).to(dev), q=torch.from_numpy(st["q"]).to(dev))
                 for st in inp.steps]
        counts = gen_step_counts(torch, kvq, lay, caches[0], quantize, steps, w, stream)
        dec_bytes = [packed_decode_bytes(lay, c) for c in counts]
        ctx_pairs = [w.batch * w.q_heads * (w.tokens + i + 1) for i in range(len(steps))]
    else:
        dec_bytes = [packed_decode_bytes(lay, [[w.n_hi, w.tokens - w.n_hi]] * w.batch)]
        ctx_pairs = [w.batch * w.q_heads * w.tokens]
    n_dec = len(dec_bytes)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def one_step(i, rec):
        """The whole hot path once: prefix quantize, then every generation
        step (append + decode), or one decode.  rec: event lists or None; a
        call is bracketed by events only where rec holds lists for it."""
        if rec is not None:
            rec["q"][i][0].record(stream)
        quantize(i)
        if rec is not None:
            rec["q"][i][1].record(stream)
        for j in range(n_dec):
            if gen:
                st = steps[j]
                if rec is not None and "a" in rec:
                    rec["a"][i][j][0].record(stream)
                kvq.append(lay, caches[0], st["k"], st["v"], st["s"], stream=stream)
                if rec is not None and "a" in rec:
                    rec["a"][i][j][1].record(stream)
            if rec is not None and "d" in rec:
                rec["d"][i][j][0].record(stream)
            decode(i, steps[j]["q"] if gen else None)
            if rec is not None and "d" in rec:
                rec["d"][i][j][1].record(stream)

    for i in range(args.warmup):
        one_step(i, None)
    torch.cuda.synchronize()
    K = args.steps
    # events bracket the quantize and every decode call of the timed steps
    # (the roofline's live durations); the appends are timed in one more step
    # after the timed region, since 512 more event markers per step would
    # lengthen the step they measure
    rec = {"q": [[ev(), ev()] for _ in range(K)],
           "d": [[[ev(), ev()] for _ in range(n_dec)] for _ in range(K)]}
    e0, e1 = ev(), ev()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        one_step(i, rec)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / K
    print(f"[bench] {K} steps: {ms_step:.3f} ms/step (wall {wall:.2f} s)", file=sys.stderr, flush=True)

    # live durations of every call in the timed steps (HIP events on `stream`)
    q_t = np.array([a.elapsed_time(b) for a, b in rec["q"]])
    d_t = np.array([[a.elapsed_time(b) for a, b in r] for r in rec["d"]])          # [K][n_dec]
    a_t = None
    if gen:
        rec_a = {"q": [[ev(), ev()]], "a": [[[ev(), ev()] for _ in range(n_dec)]]}
        one_step(0, rec_a)
        torch.cuda.synchronize()
        a_t = np.array([[a.elapsed_time(b) for a, b in r] for r in rec_a["a"]])
    dec_total_bytes = float(sum(dec_bytes))
    dec_mean_ms = float(d_t.mean())
    dec_gbs = dec_total_bytes / n_dec / (dec_mean_ms * 1e-3) / 1e9   # bytes per launch / mean duration
    if not gen and R == 1:
        print("[bench] note: decode reads the cache the same step's quantize wrote", file=sys.stderr)
    q_bytes = quantize_bytes(w, lay)
    q_med = float(np.median(q_t))
    q_gbs = q_bytes / (q_med * 1e-3) / 1e9

    # workloads without generation steps: decode alone over rotating replicas (HBM reads)
    dec_rot = None
    if not gen and R > 1:
        for i in range(3):
            decode(i)
        dm, dp10, dp90 = _timed(torch, stream, decode, args.decode_iters)
        dec_rot = dict(ms=dm, ms_p10=dp10, ms_p90=dp90, replicas=R,
                       gbs=round(dec_bytes[0] / (dm * 1e-3) / 1e9, 1))
        dec_gbs = dec_bytes[0] / (dm * 1e-3) / 1e9
        dec_mean_ms = dm

    decode_info = dict(calls=int(d_t.size), ms_mean=dec_mean_ms, ms_median=float(np.median(d_t)),
                       ms_p10=float(np.percentile(d_t, 10)), ms_p90=float(np.percentile(d_t, 90)),
                       bytes_per_call=dec_total_bytes / n_dec, gbs=round(dec_gbs, 1),
                       frac_hbm=round(dec_gbs / HBM_PEAK_GBS, 4),
                       ctx_tokens_per_s_per_qhead=sum(ctx_pairs) / (float(d_t.mean(axis=0).sum()) * 1e-3),
                       ctx_tokens_per_s_per_kvhead=sum(ctx_pairs) / (w.q_heads // w.kv_heads)
                       / (float(d_t.mean(axis=0).sum()) * 1e-3))
    if dec_rot:
        decode_info["rotating_replicas"] = dec_rot
    quant_info = dict(ms=q_med, ms_p10=float(np.percentile(q_t, 10)), ms_p90=float(np.percentile(q_t, 90)),
                      bytes=q_bytes, gbs=round(q_gbs, 1), frac_hbm=round(q_gbs / HBM_PEAK_GBS, 4))
    khash = kernel_hash(*DECODE_SOURCES)
    roof = dict(bound="hbm", achieved=round(dec_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(dec_gbs / HBM_PEAK_GBS, 4),
                traffic=measured_traffic("decode", khash, w.name),
                kernel="kvq_decode_attn (both tier pools in one kernel + merge)",
                bytes_per_launch=round(dec_total_bytes / n_dec), launch_ms=round(dec_mean_ms, 5))
    read_gbs = stream_read_gbs(torch, kvq, dev, stream)
    roof["achievable_read_gbs"] = round(read_gbs, 1)
    roof["frac_of_achievable"] = round(roof["achieved"] / read_gbs, 4)

    res = {
        "metric": "decode-attn over packed KV: context tokens/s per head & HBM GB/s; quantize GB/s",
        "value": sum(ctx_pairs) / (ms_step * 1e-3),
        "unit": "decode-attention context tokens/s per query head (whole step: prefix quantize"
                + (f" + {n_dec} x (append + decode))" if gen else " + decode)"),
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 operands (MFMA), f32 accumulate",
        "data": "synthetic (seeded N(0,1) K/V with 4 outlier key channels x10, lognormal scores)",
        "config": {"workload": w.name, "batch": w.batch, "kv_heads": w.kv_heads, "q_heads": w.q_heads,
                   "head_dim": w.head_dim, "context": w.tokens, "append_steps": w.append_steps,
                   "levels": [w.levels_hi, w.levels_lo], "group": w.group, "n_hi": w.n_hi},
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": decode_info,
        "quantize": quant_info,
    }
    if gen:
        res["append"] = dict(calls=int(a_t.size), ms_median=float(np.median(a_t)),
                             ms_p90=float(np.percentile(a_t, 90)),
                             timed="HIP events in one more step after the timed region")
    print(json.dumps(res))


if __name__ == "__main__":
    main()
