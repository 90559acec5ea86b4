"""C-ABI boundary: the library loads, exports every declared entry point, and
validates arguments on the host (no GPU is touched on any path here)."""
import ctypes
import os
import re
import subprocess

import pytest

from mixed_precision_kv_amd import kvq, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")

FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation first


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^;(]*\b(kvq_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert {"kvq_layout_init", "kvq_workspace_bytes", "kvq_status_str", "kvq_quantize",
            "kvq_append", "kvq_decode_attn", "kvq_multi_workspace_bytes",
            "kvq_decode_attn_multi", "kvq_stream_read", "kvq_decode_attn_mass",
            "kvq_set_channel_order", "kvq_decode_attn_noalloc"} <= set(names)
    L = kvq.lib()
    for n in names:
        assert hasattr(L, n), n


def test_structs_match_header(tmp_path):
    """Field offsets and sizes of the ctypes structs equal the C compiler's."""
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kvq.h"', 'int main(void){']
    for struct, cls in (("kvq_config", kvq.KvqConfig), ("kvq_layout", kvq.KvqLayout)):
        lines.append(f'printf("{struct} %zu\\n", sizeof({struct}));')
        for name, _ in cls._fields_:
            lines.append(f'printf("{struct}.{name} %zu\\n", offsetof({struct}, {name}));')
    lines.append("return 0;}")
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                    check=True).stdout.splitlines())
    for struct, cls in (("kvq_config", kvq.KvqConfig), ("kvq_layout", kvq.KvqLayout)):
        assert int(got[struct]) == ctypes.sizeof(cls)
        for name, _ in cls._fields_:
            assert int(got[f"{struct}.{name}"]) == getattr(cls, name).offset, name


@pytest.mark.parametrize("w", synth.CONFIGS + [synth.W_SKVQ], ids=lambda w: w.name)
def test_layout_of_every_workload(w):
    lay = kvq.layout_init(kvq.config_for(w))
    assert lay.total_bytes > 0
    offs = [lay.counters, lay.tokmap, lay.sorted, *lay.k_words, *lay.k_meta, *lay.v_words,
            *lay.v_meta, lay.sparse, lay.k_win, lay.v_win]
    assert all(o % 256 == 0 for o in offs)
    assert kvq.workspace_bytes(lay, kvq.OP_QUANTIZE, w.tokens) > 0
    assert kvq.workspace_bytes(lay, kvq.OP_DECODE, w.capacity) > 0
    if w.mode == "tiered":
        assert lay.nv[0] == {6: 12, 8: 10}[w.levels_hi]
        assert lay.kw[1] == {5: 10, 6: 11}[w.levels_lo]
    else:
        assert lay.nv[0] == 16 and lay.vnv == 20 and lay.win_cap == 255


def _cfg(**kw):
    c = kvq.config_for(synth.W_SINGLE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), 2), (dict(q_heads=8), 2), (dict(levels_hi=2), 2), (dict(levels_lo=17), 2), (dict(levels_hi=9), 2),
    (dict(levels_lo=9), 2),
    (dict(group=48), 2), (dict(capacity=0), 1), (dict(batch=0), 1), (dict(mode=7), 1),
    (dict(cap_hi=100, cap_lo=100), 1), (dict(cap_hi=5000), 1),
    (dict(reorder=2), 1), (dict(clip=-0.5), 1), (dict(clip=1.5), 1), (dict(clip=float("nan")), 1),
    (dict(rope_theta=0.5), 1), (dict(rope_theta=-1.0), 1), (dict(rope_theta=float("inf")), 1),
    (dict(rope_theta=10000.0, reorder=1), 2),
])
def test_layout_rejects(kw, status):
    with pytest.raises(kvq.KvqError) as e:
        kvq.layout_init(_cfg(**kw))
    assert e.value.status == status


def test_kchan_rejects_unsupported():
    w = synth.W_KCHAN
    for kw in (dict(k_block=64), dict(v_levels=5), dict(window=600), dict(sparse_per_vec=9),
               dict(reorder=1), dict(clip=0.9), dict(rope_theta=10000.0)):
        c = kvq.config_for(w)
        for k, v in kw.items():
            setattr(c, k, v)
        with pytest.raises(kvq.KvqError) as e:
            kvq.layout_init(c)
        assert e.value.status == 2


def test_workspace_bad_args():
    lay = kvq.layout_init(_cfg())
    assert kvq.workspace_bytes(lay, kvq.OP_DECODE, 0) == 0
    assert kvq.workspace_bytes(lay, kvq.OP_DECODE, lay.cfg.capacity + 1) == 0
    assert kvq.workspace_bytes(lay, 9, 16) == 0


def _quant(lay, **over):
    a = dict(cache=FAKE, k=FAKE, v=FAKE, strides=(4096 * 128, 128, 128), scores=FAKE, T=4096,
             n_hi=2048, ranks_out=None, ws=FAKE, ws_bytes=1 << 40, stream=0)
    a.update(over)
    kvq.quantize(lay, a["cache"], a["k"], a["v"], a["scores"], a["T"], a["n_hi"], a["ranks_out"],
                 a["ws"], a["ws_bytes"], strides=a["strides"], stream=a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(cache=0), 1), (dict(k=0), 1), (dict(v=FAKE + 4), 1), (dict(scores=0), 1),
    (dict(T=0), 1), (dict(T=4097), 3), (dict(n_hi=-1), 1), (dict(n_hi=4097), 1),
    (dict(strides=(4096 * 128, 100, 128)), 1), (dict(strides=(-8, 128, 128)), 1),
    (dict(ws=0), 4), (dict(ws_bytes=1000), 4), (dict(ranks_out=FAKE + 2), 1),
])
def test_quantize_validation(over, status):
    lay = kvq.layout_init(_cfg())
    with pytest.raises(kvq.KvqError) as e:
        _quant(lay, **over)
    assert e.value.status == status


def test_layout_unit_count_limit():
    """(sequence, KV head) units index the kernels' second grid dimension,
    which holds 65536 workgroups: one unit more is refused by the layout."""
    kvq.layout_init(_cfg(batch=65536))
    with pytest.raises(kvq.KvqError) as e:
        kvq.layout_init(_cfg(batch=65537))
    assert e.value.status == 2
    with pytest.raises(kvq.KvqError) as e:
        kvq.layout_init(_cfg(batch=16385, kv_heads=4, q_heads=16))
    assert e.value.status == 2


def test_quantize_longest_ranked_sequence():
    """The rank kernels take sequences of up to 262144 tokens; one more is
    refused before any launch, whatever the capacity."""
    lay = kvq.layout_init(_cfg(capacity=262145, cap_hi=0, cap_lo=0))
    strides = (262145 * 128, 128, 128)
    with pytest.raises(kvq.KvqError) as e:
        _quant(lay, T=262145, n_hi=131072, strides=strides)
    assert e.value.status == 2
    with pytest.raises(kvq.KvqError) as e:            # the limit itself passes validation
        _quant(lay, T=262144, n_hi=131072, strides=strides, ws=0)
    assert e.value.status == 4                        # (stopped at the missing workspace)


def test_quantize_capacity_per_pool():
    c = _cfg(capacity=4096, cap_hi=2048, cap_lo=2048)
    lay = kvq.layout_init(c)
    with pytest.raises(kvq.KvqError) as e:
        _quant(lay, n_hi=2049)
    assert e.value.status == 3


def test_append_validation():
    lay = kvq.layout_init(_cfg())
    for args in ((0, FAKE, FAKE, FAKE), (FAKE, 0, FAKE, FAKE), (FAKE, FAKE, FAKE + 8, FAKE)):
        with pytest.raises(kvq.KvqError) as e:
            kvq.append(lay, *args, stream=0)
        assert e.value.status == 1
    lay5 = kvq.layout_init(kvq.config_for(synth.W_KCHAN))
    with pytest.raises(kvq.KvqError) as e:
        kvq.append(lay5, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == 2


@pytest.mark.parametrize("over,status", [
    (dict(cache=0), 1), (dict(q=FAKE + 2), 1), (dict(out=0), 1), (dict(scale=0.0), 1),
    (dict(scale=float("nan")), 1), (dict(max_len=0), 1), (dict(max_len=4097), 3),
    (dict(ws=0), 4), (dict(ws_bytes=64), 4),
])
def test_decode_validation(over, status):
    lay = kvq.layout_init(_cfg())
    a = dict(cache=FAKE, q=FAKE, scale=0.088, max_len=4096, out=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(over)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn(lay, a["cache"], a["q"], a["scale"], a["max_len"], a["out"], a["ws"],
                        ws_bytes=a["ws_bytes"], stream=0)
    assert e.value.status == status


@pytest.mark.parametrize("over,status", [
    (dict(cache=0), 1), (dict(q=FAKE + 2), 1), (dict(out=0), 1), (dict(lse=FAKE + 2), 1),
    (dict(n_queries=0), 1), (dict(n_queries=4097), 1), (dict(scale=-1.0), 1),
    (dict(max_len=0), 1), (dict(max_len=4097), 3), (dict(ws=0), 4), (dict(ws_bytes=64), 4),
])
def test_decode_multi_validation(over, status):
    lay = kvq.layout_init(_cfg())
    a = dict(cache=FAKE, q=FAKE, n_queries=8, scale=0.088, max_len=4096, out=FAKE, lse=None,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(over)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_multi(lay, a["cache"], a["q"], a["n_queries"], a["scale"], a["max_len"],
                              a["out"], a["lse"], a["ws"], ws_bytes=a["ws_bytes"], stream=0)
    assert e.value.status == status


def test_decode_multi_workspace_and_mode():
    lay = kvq.layout_init(_cfg())
    one = kvq.multi_workspace_bytes(lay, 4, 4096)
    assert one > 0 and kvq.multi_workspace_bytes(lay, 5, 4096) == 2 * one   # four queries a group
    assert kvq.multi_workspace_bytes(lay, 0, 4096) == 0
    assert kvq.multi_workspace_bytes(lay, 4, 4097) == 0
    lay5 = kvq.layout_init(kvq.config_for(synth.W_KCHAN))
    assert kvq.multi_workspace_bytes(lay5, 4, 1024) == 0
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_multi(lay5, FAKE, FAKE, 4, 0.088, 1024, FAKE, None, FAKE, ws_bytes=1 << 40,
                              stream=0)
    assert e.value.status == 2


@pytest.mark.parametrize("over,status", [
    (dict(cache=0), 1), (dict(q=FAKE + 2), 1), (dict(out=0), 1), (dict(mass=0), 1),
    (dict(mass=FAKE + 2), 1), (dict(scale=0.0), 1), (dict(max_len=0), 1), (dict(max_len=4097), 3),
    (dict(ws=0), 4), (dict(ws_bytes=64), 4),
])
def test_decode_mass_validation(over, status):
    lay = kvq.layout_init(_cfg())
    a = dict(cache=FAKE, q=FAKE, scale=0.088, max_len=4096, out=FAKE, mass=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(over)
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_mass(lay, a["cache"], a["q"], a["scale"], a["max_len"], a["out"], a["mass"],
                             a["ws"], ws_bytes=a["ws_bytes"], stream=0)
    assert e.value.status == status


def test_decode_mass_workspace_and_mode():
    lay = kvq.layout_init(_cfg())
    plain = kvq.workspace_bytes(lay, kvq.OP_DECODE, 4096)
    extra = kvq.workspace_bytes(lay, kvq.OP_DECODE_MASS, 4096) - plain
    U = lay.cfg.batch * lay.cfg.kv_heads
    assert extra == U * 4 * (lay.cap[0] + lay.cap[1]) * 4 + U * 4 * 8
    lay5 = kvq.layout_init(kvq.config_for(synth.W_KCHAN))
    assert kvq.workspace_bytes(lay5, kvq.OP_DECODE_MASS, 1024) == 0
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_mass(lay5, FAKE, FAKE, 0.088, 1024, FAKE, FAKE, FAKE, ws_bytes=1 << 40, stream=0)
    assert e.value.status == 2


@pytest.mark.parametrize("buf,nbytes,sink,nwg", [
    (0, 1024, FAKE, 8), (FAKE + 8, 1024, FAKE, 8), (FAKE, 1000, FAKE, 8), (FAKE, 0, FAKE, 8),
    (FAKE, 1024, 0, 8), (FAKE, 1024, FAKE + 2, 8), (FAKE, 1024, FAKE, 0), (FAKE, 1024, FAKE, 65537),
])
def test_stream_read_validation(buf, nbytes, sink, nwg):
    st = kvq.lib().kvq_stream_read(buf, nbytes, sink, nwg, None)
    assert st == 1


def test_status_strings():
    L = kvq.lib()
    for s in range(6):
        assert L.kvq_status_str(s)
    assert L.kvq_status_str(99) == b"unknown status"


def test_channel_order_layout_and_workspace():
    """reorder = 1 adds the [2][Hkv][D] byte orders to the cache and nothing
    to any workspace (decode reads q through the stored order); clipping
    alone adds nothing."""
    plain = kvq.layout_init(_cfg())
    lay = kvq.layout_init(_cfg(reorder=1, clip=0.9))
    assert plain.chan_order == 0
    assert lay.chan_order % 256 == 0 and lay.chan_order + 2 * 128 <= lay.total_bytes
    assert lay.total_bytes == plain.total_bytes + 256
    clipped = kvq.layout_init(_cfg(clip=0.5))
    assert clipped.total_bytes == plain.total_bytes and clipped.chan_order == 0
    for op in (kvq.OP_QUANTIZE, kvq.OP_DECODE, kvq.OP_DECODE_MASS):
        assert kvq.workspace_bytes(lay, op, 4096) == kvq.workspace_bytes(plain, op, 4096)
    assert kvq.multi_workspace_bytes(lay, 6, 4096) == kvq.multi_workspace_bytes(plain, 6, 4096)


def test_set_channel_order_validation():
    import numpy as np
    lay = kvq.layout_init(_cfg(reorder=1))
    ident = np.tile(np.arange(128, dtype=np.int32), (2, 1, 1))
    bad_dup = ident.copy()
    bad_dup[1, 0, 5] = 6
    bad_range = ident.copy()
    bad_range[0, 0, 0] = 128
    bad_neg = ident.copy()
    bad_neg[0, 0, 7] = -1
    for o in (bad_dup, bad_range, bad_neg):
        with pytest.raises(kvq.KvqError) as e:
            kvq.set_channel_order(lay, FAKE, o, stream=0)
        assert e.value.status == 1
    with pytest.raises(kvq.KvqError) as e:                 # cache laid out without orders
        kvq.set_channel_order(kvq.layout_init(_cfg()), FAKE, ident, stream=0)
    assert e.value.status == 2
    with pytest.raises(kvq.KvqError) as e:                 # misaligned cache
        kvq.set_channel_order(lay, FAKE + 8, ident, stream=0)
    assert e.value.status == 1
    with pytest.raises(ValueError):                        # too few entries for the layout
        kvq.set_channel_order(lay, FAKE, ident[:1], stream=0)


def test_noalloc_decode_validation():
    """The allocation-free decode rejects bad arguments, and partials beyond
    its fixed 16 MiB array (512 x 8 units need at least 17.3 MB), on the
    host before any launch."""
    lay = kvq.layout_init(_cfg())
    for args, status in (((0, FAKE, 0.088, 64, FAKE), 1), ((FAKE, FAKE + 2, 0.088, 64, FAKE), 1),
                         ((FAKE, FAKE, 0.0, 64, FAKE), 1), ((FAKE, FAKE, 0.088, 0, FAKE), 1),
                         ((FAKE, FAKE, 0.088, lay.cfg.capacity + 1, FAKE), 3)):
        with pytest.raises(kvq.KvqError) as e:
            kvq.decode_attn_noalloc(lay, args[0], args[1], args[2], args[3], args[4], stream=0)
        assert e.value.status == status
    big = kvq.layout_init(kvq.config_for(synth.W_LLAMA.shrink(name="huge", batch=512, tokens=64)))
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_noalloc(big, FAKE, FAKE, 0.088, 64, FAKE, stream=0)
    assert e.value.status == 4


def test_rope_layout_and_multi_query_unsupported():
    """Pre-RoPE keys add the per-pool slot positions to the layout; the
    multi-query entry point refuses such a cache on the host."""
    w = synth.W_ROPE.shrink(name="rope_small", batch=2, kv_heads=2, q_heads=8, tokens=1000)
    lay = kvq.layout_init(kvq.config_for(w))
    plain = kvq.layout_init(kvq.config_for(w.shrink(rope_theta=0.0)))
    assert plain.slot_pos[0] == plain.slot_pos[1] == 0
    assert lay.slot_pos[0] > 0 and lay.slot_pos[1] > lay.slot_pos[0] and lay.slot_pos[0] % 256 == 0
    assert lay.total_bytes - plain.total_bytes >= 4 * 2 * (lay.cap[0] + lay.cap[1])
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attn_multi(lay, FAKE, FAKE, 4, 0.088, 1000, FAKE, None, FAKE, 1 << 30, stream=0)
    assert e.value.status == 2
