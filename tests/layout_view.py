"""Canonical views of a cache buffer, read with the index formulas documented
in include/kvq.h (test code; independent of the library's kernels).

Canonical forms match the oracle: row key words [n][kw], column value words
[rows][D], (scale, zero) as fp16 arrays [n][D/G], token map, counters."""
import numpy as np


def _u32(buf, off, n):
    return np.frombuffer(buf, dtype=np.uint32, count=n, offset=off)


def counters(buf, lay):
    B = lay.cfg.batch
    return np.frombuffer(buf, dtype=np.int32, count=B * 4, offset=lay.counters).reshape(B, 4)


def tokmap(buf, lay):
    B, cap = lay.cfg.batch, lay.cfg.capacity
    return _u32(buf, lay.tokmap, B * cap).reshape(B, cap)


def sorted_scores(buf, lay):
    B, cap = lay.cfg.batch, lay.cfg.capacity
    return np.frombuffer(buf, dtype=np.float32, count=B * cap, offset=lay.sorted).reshape(B, cap)


def _tile_rows(arr_u32, U, tiles, width):
    """[U][tiles][width][16] -> [U][tiles*16][width]."""
    return arr_u32.reshape(U, tiles, width, 16).transpose(0, 1, 3, 2).reshape(U, tiles * 16, width)


def _split_meta(m):
    scale = (m & 0xFFFF).astype(np.uint16).view(np.float16)
    zero = (m >> 16).astype(np.uint16).view(np.float16)
    return scale, zero


def tiered_pool(buf, lay, p):
    """Canonical arrays of pool p for every unit u = b*Hkv + h (all capacity slots)."""
    c = lay.cfg
    U = c.batch * c.kv_heads
    D = c.head_dim
    NG = D // c.group
    tiles, kw, vrows = lay.tiles[p], lay.kw[p], lay.vrows[p]
    kwd = _tile_rows(_u32(buf, lay.k_words[p], U * tiles * kw * 16), U, tiles, kw)
    km = _tile_rows(_u32(buf, lay.k_meta[p], U * tiles * NG * 16), U, tiles, NG)
    vm = _tile_rows(_u32(buf, lay.v_meta[p], U * tiles * NG * 16), U, tiles, NG)
    vwd = _u32(buf, lay.v_words[p], U * vrows * D).reshape(U, vrows, D)
    ks, kz = _split_meta(km)
    vs, vz = _split_meta(vm)
    return dict(k_words=kwd, k_scale=ks, k_zero=kz, v_words=vwd, v_scale=vs, v_zero=vz)


def kchan_unit_arrays(buf, lay):
    c = lay.cfg
    U = c.batch * c.kv_heads
    D = c.head_dim
    NG = D // c.v_group
    tiles, kw, vrows = lay.tiles[0], lay.kw[0], lay.vrows[0]
    kwd = _tile_rows(_u32(buf, lay.k_words[0], U * tiles * kw * 16), U, tiles, kw)
    km = _u32(buf, lay.k_meta[0], U * lay.kblocks * D).reshape(U, lay.kblocks, D)
    sp = _u32(buf, lay.sparse, U * c.capacity * c.sparse_per_vec).reshape(U, c.capacity, c.sparse_per_vec)
    vwd = _u32(buf, lay.v_words[0], U * vrows * D).reshape(U, vrows, D)
    vm = _tile_rows(_u32(buf, lay.v_meta[0], U * tiles * NG * 16), U, tiles, NG)
    kwin = np.frombuffer(buf, dtype=np.float16, count=U * lay.win_cap * D, offset=lay.k_win).reshape(U, lay.win_cap, D)
    vwin = np.frombuffer(buf, dtype=np.float16, count=U * lay.win_cap * D, offset=lay.v_win).reshape(U, lay.win_cap, D)
    ks, kz = _split_meta(km)
    vs, vz = _split_meta(vm)
    return dict(k_words=kwd, k_scale=ks, k_zero=kz, sparse=sp, v_words=vwd, v_scale=vs, v_zero=vz,
                k_win=kwin, v_win=vwin)


def slot_positions(buf, lay, p):
    """Token position of every slot of pool p, [B][cap[p]] (pre-RoPE keys)."""
    B, cap = lay.cfg.batch, lay.cap[p]
    return np.frombuffer(buf, dtype=np.int32, count=B * cap, offset=lay.slot_pos[p]).reshape(B, cap)
