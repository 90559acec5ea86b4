"""Thin ctypes binding of libkvq.so (the C ABI in include/kvq.h).

Argument marshalling only: every step of quantize, append and decode runs in
the library's HIP kernels.  Tensors are passed by device pointer; PyTorch is
used for device memory and for the current HIP stream, nothing else.  If the
library has not been built, every entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

MODE_TIERED, MODE_KCHAN = 0, 1
OP_QUANTIZE, OP_DECODE, OP_DECODE_MASS = 0, 1, 2
STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_ARG", 2: "KVQ_ERR_UNSUPPORTED", 3: "KVQ_ERR_CAPACITY",
          4: "KVQ_ERR_WORKSPACE", 5: "KVQ_ERR_LAUNCH"}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class KvqConfig(ctypes.Structure):
    _fields_ = [(n, _i32) for n in (
        "mode", "batch", "kv_heads", "q_heads", "head_dim", "capacity",
        "levels_hi", "levels_lo", "group", "cap_hi", "cap_lo",
        "k_levels", "k_block", "v_levels", "v_group", "window", "sparse_per_vec",
        "reorder")] + [("clip", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class KvqLayout(ctypes.Structure):
    _fields_ = [
        ("cfg", KvqConfig),
        ("nv", _i32 * 2), ("kw", _i32 * 2), ("cap", _i32 * 2), ("tiles", _i32 * 2),
        ("vrows", _i32 * 2),
        ("kblocks", _i32), ("win_cap", _i32), ("vnv", _i32), ("reserved", _i32),
        ("counters", _i64), ("tokmap", _i64), ("sorted", _i64),
        ("k_words", _i64 * 2), ("k_meta", _i64 * 2), ("v_words", _i64 * 2), ("v_meta", _i64 * 2),
        ("sparse", _i64), ("k_win", _i64), ("v_win", _i64),
        ("chan_order", _i64),
        ("slot_pos", _i64 * 2),
        ("total_bytes", _i64),
    ]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixed_precision_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, cp = ctypes.c_void_p, ctypes.POINTER
        L.kvq_layout_init.argtypes = [cp(KvqConfig), cp(KvqLayout)]
        L.kvq_layout_init.restype = ctypes.c_int
        L.kvq_workspace_bytes.argtypes = [cp(KvqLayout), _i32, _i32]
        L.kvq_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_status_str.argtypes = [ctypes.c_int]
        L.kvq_status_str.restype = ctypes.c_char_p
        L.kvq_quantize.argtypes = [cp(KvqLayout), vp, vp, vp, _i64, _i64, _i64, vp, _i32, _i32, vp,
                                   vp, ctypes.c_size_t, vp]
        L.kvq_quantize.restype = ctypes.c_int
        L.kvq_append.argtypes = [cp(KvqLayout), vp, vp, vp, vp, vp]
        L.kvq_append.restype = ctypes.c_int
        L.kvq_decode_attn.argtypes = [cp(KvqLayout), vp, vp, ctypes.c_float, _i32, vp, vp,
                                      ctypes.c_size_t, vp]
        L.kvq_decode_attn.restype = ctypes.c_int
        L.kvq_multi_workspace_bytes.argtypes = [cp(KvqLayout), _i32, _i32]
        L.kvq_multi_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_decode_attn_multi.argtypes = [cp(KvqLayout), vp, vp, _i32, ctypes.c_float, _i32, vp, vp,
                                            vp, ctypes.c_size_t, vp]
        L.kvq_decode_attn_multi.restype = ctypes.c_int
        L.kvq_decode_attn_mass.argtypes = [cp(KvqLayout), vp, vp, ctypes.c_float, _i32, vp, vp, vp,
                                           ctypes.c_size_t, vp]
        L.kvq_decode_attn_mass.restype = ctypes.c_int
        L.kvq_set_channel_order.argtypes = [cp(KvqLayout), vp, vp, vp]
        L.kvq_set_channel_order.restype = ctypes.c_int
        L.kvq_decode_attn_noalloc.argtypes = [cp(KvqLayout), vp, vp, ctypes.c_float, _i32, vp, vp]
        L.kvq_decode_attn_noalloc.restype = ctypes.c_int
        L.kvq_stream_read.argtypes = [vp, ctypes.c_size_t, vp, _i32, vp]
        L.kvq_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(st: int, what: str):
    if st != 0:
        raise KvqError(st, what)


def config_for(w) -> KvqConfig:
    """kvq_config for a synth.Workload (capacity covers its append steps)."""
    c = KvqConfig()
    c.mode = MODE_TIERED if w.mode == "tiered" else MODE_KCHAN
    c.batch, c.kv_heads, c.q_heads, c.head_dim = w.batch, w.kv_heads, w.q_heads, w.head_dim
    c.capacity = w.capacity
    if c.mode == MODE_TIERED:
        c.levels_hi, c.levels_lo, c.group = w.levels_hi, w.levels_lo, w.group
        c.cap_hi = min(w.capacity, w.n_hi + w.append_steps)
        c.cap_lo = min(w.capacity, w.tokens - w.n_hi + w.append_steps)
        c.reorder = 1 if w.reorder else 0
        c.clip = w.clip
        c.rope_theta = getattr(w, "rope_theta", 0.0)
    else:
        c.k_levels, c.k_block, c.v_levels, c.v_group = w.k_levels, w.k_block, w.v_levels, w.v_group
        c.window, c.sparse_per_vec = w.window, w.sparse_per_vec
    return c


def layout_init(cfg: KvqConfig) -> KvqLayout:
    lay = KvqLayout()
    _check(lib().kvq_layout_init(ctypes.byref(cfg), ctypes.byref(lay)), "kvq_layout_init")
    return lay


def workspace_bytes(lay: KvqLayout, op: int, max_len: int) -> int:
    return int(lib().kvq_workspace_bytes(ctypes.byref(lay), op, max_len))


def set_channel_order(lay, cache, order, stream=None):
    """order: host int32 array [2][Hkv][D] (keys, values); entry p of a row is
    the channel stored at position p."""
    import numpy as np
    o = np.ascontiguousarray(order, dtype=np.int32)
    want = (2, lay.cfg.kv_heads, lay.cfg.head_dim)
    if o.shape != want:                     # the library reads exactly this many entries
        raise ValueError(f"channel order shape {o.shape}, expected {want}")
    st = lib().kvq_set_channel_order(ctypes.byref(lay), _ptr(cache), o.ctypes.data, _stream(stream))
    _check(st, "kvq_set_channel_order")


def quantize(lay, cache, k, v, scores, T, n_hi, ranks_out=None, ws=None, ws_bytes=None,
             strides=None, stream=None):
    """k, v: fp16 [B][T][Hkv][D] device tensors (or any strides with d contiguous)."""
    if strides is None:
        assert k.stride() == v.stride() and k.stride(3) == 1
        strides = (k.stride(0), k.stride(1), k.stride(2))
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().kvq_quantize(ctypes.byref(lay), _ptr(cache), _ptr(k), _ptr(v), strides[0],
                            strides[1], strides[2], _ptr(scores), T, n_hi, _ptr(ranks_out),
                            _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "kvq_quantize")


def append(lay, cache, k_new, v_new, score_new, stream=None):
    st = lib().kvq_append(ctypes.byref(lay), _ptr(cache), _ptr(k_new), _ptr(v_new),
                          _ptr(score_new), _stream(stream))
    _check(st, "kvq_append")


def decode_attn(lay, cache, q, scale, max_len, out, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().kvq_decode_attn(ctypes.byref(lay), _ptr(cache), _ptr(q), float(scale), max_len,
                               _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "kvq_decode_attn")


def decode_attn_noalloc(lay, cache, q, scale, max_len, out, stream=None):
    """kvq_decode_attn with the library's fixed device array as workspace."""
    st = lib().kvq_decode_attn_noalloc(ctypes.byref(lay), _ptr(cache), _ptr(q), float(scale), max_len,
                                       _ptr(out), _stream(stream))
    _check(st, "kvq_decode_attn_noalloc")


def multi_workspace_bytes(lay: KvqLayout, n_queries: int, max_len: int) -> int:
    return int(lib().kvq_multi_workspace_bytes(ctypes.byref(lay), n_queries, max_len))


def decode_attn_multi(lay, cache, q, n_queries, scale, max_len, out, lse, ws, ws_bytes=None,
                      stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().kvq_decode_attn_multi(ctypes.byref(lay), _ptr(cache), _ptr(q), n_queries, float(scale),
                                     max_len, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
                                     _stream(stream))
    _check(st, "kvq_decode_attn_multi")


def stream_read(buf, sink, n_workgroups, stream=None):
    """Measurement aid: read every byte of `buf` once on the device."""
    st = lib().kvq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), n_workgroups,
                               _stream(stream))
    _check(st, "kvq_stream_read")


def decode_attn_mass(lay, cache, q, scale, max_len, out, mass, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().kvq_decode_attn_mass(ctypes.byref(lay), _ptr(cache), _ptr(q), float(scale), max_len,
                                    _ptr(out), _ptr(mass), _ptr(ws), ws_bytes, _stream(stream))
    _check(st, "kvq_decode_attn_mass")
