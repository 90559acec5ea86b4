"""The allocation-free decode entry point (kvq_decode_attn_noalloc), called
through the C ABI, against kvq_decode_attn on the same cache: two calls in a
row, the second on a smaller input, and per-channel keys.  The two entry
points run the same kernels with the same chunk split, so their fp16
outputs must be identical (stronger than the 2e-3 bar against the
oracle, which the decode tests already check)."""
import numpy as np
import pytest

from mixed_precision_kv_amd import kvq, synth
from gpu_harness import GpuRun, log, to_dev

pytestmark = pytest.mark.gpu


def _both(run, q_np, max_len):
    import torch
    q = to_dev(q_np)
    ref = torch.empty_like(q)
    out = torch.full_like(q, float("nan"))
    kvq.decode_attn(run.lay, run.cache, q, float(run.scale), max_len, ref, run.wsd)
    kvq.decode_attn_noalloc(run.lay, run.cache, q, float(run.scale), max_len, out)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    (synth.W_LLAMA.shrink(name="noalloc_big", batch=4, kv_heads=4, q_heads=16, tokens=6001),
     synth.W_LLAMA.shrink(name="noalloc_small", batch=2, kv_heads=2, q_heads=8, tokens=777)),
    (synth.W_LONG.shrink(name="noalloc_long", batch=1, kv_heads=8, q_heads=32, tokens=20000),
     synth.W_SINGLE.shrink(name="noalloc_tiny", tokens=100)),
    (synth.W_KCHAN.shrink(name="noalloc_kchan", batch=2, kv_heads=4, q_heads=16, tokens=5000),
     synth.W_KCHAN.shrink(name="noalloc_kchan_small", batch=1, kv_heads=2, q_heads=8, tokens=300)),
], ids=["tiered", "long_then_tiny", "kchan"])
def test_noalloc_matches_decode(first, second):
    for w in (first, second):
        log(f"case {w.name} B{w.batch} H{w.kv_heads} T{w.tokens}")
        inp = synth.make_inputs(w)
        run = GpuRun(w, inp, want_ranks=False)
        run.quantize()
        ref, out = _both(run, inp.q, w.tokens)
        assert np.isfinite(ref.astype(np.float32)).all()
        assert np.array_equal(out.view(np.uint16), ref.view(np.uint16)), w.name


def test_noalloc_after_appends():
    """Generation steps: each step's decode through both entry points."""
    w = synth.W_APPEND.shrink(name="noalloc_append", batch=3, kv_heads=2, q_heads=8, tokens=500, append_steps=4)
    log(f"case {w.name}")
    inp = synth.make_inputs(w)
    run = GpuRun(w, inp, want_ranks=False)
    run.quantize()
    for i, st in enumerate(inp.steps):
        run.append(st)
        ref, out = _both(run, st["q"], w.capacity)
        assert np.array_equal(out.view(np.uint16), ref.view(np.uint16)), f"step {i}"
