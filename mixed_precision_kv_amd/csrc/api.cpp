// Host side of the C ABI: layout, workspace sizing, argument validation and
// dispatch to the kernel launchers.  Nothing here touches the GPU except the
// launchers, which run only after every argument has been checked.
#include <string.h>

#include "common.h"
#include "internal.h"
#include "tiling.h"

namespace kvq {

static int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

static bool levels_ok(int L) { return L >= 3 && L <= 16; }
static bool decode_levels_ok(int L) { return L >= 3 && L <= 8; }
static bool group_ok(int G) { return G == 32 || G == 64 || G == 128; }

int decode_chunks(const kvq_layout* L, int max_len, int* nch0, int* nch1) {
  if (L->cfg.mode == KVQ_MODE_TIERED) {
    int c0 = L->cap[0] < max_len ? L->cap[0] : max_len;
    int c1 = L->cap[1] < max_len ? L->cap[1] : max_len;
    // workspace bound: the finest split, one macro tile per chunk
    *nch0 = ceil_div(c0, macro_tile_slots(L->cfg.levels_hi));
    *nch1 = ceil_div(c1, macro_tile_slots(L->cfg.levels_lo));
  } else {
    int nq = kchan_nq(L, max_len);
    *nch0 = ceil_div(nq, decode_chunk_kchan(L));
    *nch1 = ceil_div(L->win_cap, kWinChunk);   // the fp16 window
  }
  return *nch0 + *nch1;
}

QuantWs quant_ws_plan(const kvq_layout* L, int T) {
  QuantWs p;
  memset(&p, 0, sizeof(p));
  const int64_t B = L->cfg.batch;
  int64_t off = 0;
  if (L->cfg.mode == KVQ_MODE_TIERED) {
    const int64_t nblk = ceil_div(T, kSortTile);
    const int64_t ld = (T + 3) & ~3;   // rows of sorted keys stay 16-byte aligned
    for (int i = 0; i < 2; ++i) { p.keys[i] = off; off = align256(off + B * ld * 4); }
    p.idx = off;    off = align256(off + B * ld * 4);
    p.segcnt = off; off = align256(off + B * nblk * 4);   // high-tier count per 1024 tokens
    p.ranks = off;  off = align256(off + B * T * 4);
    for (int i = 0; i < 2; ++i) { p.inv[i] = off; off = align256(off + B * (int64_t)L->cap[i] * 4); }
  }
  p.total = (size_t)(off > 256 ? off : 256);
  return p;
}

}  // namespace kvq

using namespace kvq;

extern "C" const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_ARG: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "capacity exceeded";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

extern "C" kvq_status kvq_layout_init(const kvq_config* cfg, kvq_layout* out) {
  if (!cfg || !out) return KVQ_ERR_ARG;
  const kvq_config c = *cfg;
  if (c.batch < 1 || c.kv_heads < 1 || c.q_heads < 1 || c.head_dim < 1 || c.capacity < 1)
    return KVQ_ERR_ARG;
  if (c.head_dim != kD || c.q_heads != kGqa * c.kv_heads) return KVQ_ERR_UNSUPPORTED;
  // kernels take the (sequence, KV head) unit as the grid's second dimension,
  // which holds at most 65536 workgroups
  if ((int64_t)c.batch * c.kv_heads > 65536 || c.capacity > (1 << 24)) return KVQ_ERR_UNSUPPORTED;
  kvq_layout L;
  memset(&L, 0, sizeof(L));
  L.cfg = c;
  const int64_t B = c.batch, U = (int64_t)c.batch * c.kv_heads, D = kD;
  int64_t off = 0;
  if (c.mode == KVQ_MODE_TIERED) {
    if (!decode_levels_ok(c.levels_hi) || !decode_levels_ok(c.levels_lo) || !group_ok(c.group))
      return KVQ_ERR_UNSUPPORTED;
    if (c.reorder != 0 && c.reorder != 1) return KVQ_ERR_ARG;
    if (!(c.clip == 0.0f || (c.clip > 0.0f && c.clip <= 1.0f))) return KVQ_ERR_ARG;
    if (!(c.rope_theta == 0.0f || (c.rope_theta > 1.0f && c.rope_theta < 1e30f))) return KVQ_ERR_ARG;
    if (c.rope_theta != 0.0f && c.reorder) return KVQ_ERR_UNSUPPORTED;   // pairs are original channels
    if (c.cap_hi < 0 || c.cap_lo < 0) return KVQ_ERR_ARG;
    L.cap[0] = c.cap_hi ? c.cap_hi : c.capacity;
    L.cap[1] = c.cap_lo ? c.cap_lo : c.capacity;
    if (L.cap[0] > c.capacity || L.cap[1] > c.capacity) return KVQ_ERR_ARG;
    if ((int64_t)L.cap[0] + L.cap[1] < c.capacity) return KVQ_ERR_ARG;
    const int lv[2] = {c.levels_hi, c.levels_lo};
    L.counters = off; off = align256(off + B * 16);
    L.tokmap = off;   off = align256(off + B * c.capacity * 4);
    L.sorted = off;   off = align256(off + B * c.capacity * 4);
    for (int p = 0; p < 2; ++p) {
      L.nv[p] = codes_per_word(lv[p]);
      L.kw[p] = ceil_div(kD, L.nv[p]);
      L.tiles[p] = ceil_div(L.cap[p], kTile);
      L.vrows[p] = ceil_div(L.cap[p], L.nv[p]);
      const int64_t ng = kD / c.group;
      L.k_words[p] = off; off = align256(off + U * L.tiles[p] * L.kw[p] * kTile * 4);
      L.k_meta[p] = off;  off = align256(off + U * L.tiles[p] * ng * kTile * 4);
      L.v_words[p] = off; off = align256(off + U * L.vrows[p] * D * 4);
      L.v_meta[p] = off;  off = align256(off + U * L.tiles[p] * ng * kTile * 4);
    }
    if (c.reorder) { L.chan_order = off; off = align256(off + 2 * (int64_t)c.kv_heads * D); }
    if (c.rope_theta != 0.0f)
      for (int p = 0; p < 2; ++p) { L.slot_pos[p] = off; off = align256(off + B * (int64_t)L.cap[p] * 4); }
  } else if (c.mode == KVQ_MODE_KCHAN) {
    if (c.reorder != 0 || c.clip != 0.0f || c.rope_theta != 0.0f) return KVQ_ERR_UNSUPPORTED;
    if (!levels_ok(c.k_levels) || !levels_ok(c.v_levels) || !group_ok(c.v_group))
      return KVQ_ERR_UNSUPPORTED;
    if (c.k_block != 128 || c.window < 0 || c.sparse_per_vec < 0 || c.sparse_per_vec > 8)
      return KVQ_ERR_UNSUPPORTED;
    L.cap[0] = c.capacity;
    L.nv[0] = codes_per_word(c.k_levels);
    L.nv[1] = codes_per_word(c.v_levels);
    L.vnv = L.nv[1];
    // decode chunks hold whole key blocks, key tiles and value word rows
    if (lcm_i(lcm_i(c.k_block, kTile), L.vnv) > 640) return KVQ_ERR_UNSUPPORTED;
    if (c.window + c.k_block - 1 > 640) return KVQ_ERR_UNSUPPORTED;
    L.kw[0] = ceil_div(kD, L.nv[0]);
    L.tiles[0] = ceil_div(c.capacity, kTile);
    L.vrows[0] = ceil_div(c.capacity, L.vnv);
    L.kblocks = ceil_div(c.capacity, c.k_block);
    L.win_cap = c.window + c.k_block - 1;
    if (L.win_cap > c.capacity) L.win_cap = c.capacity;
    const int64_t ng = kD / c.v_group;
    L.counters = off; off = align256(off + B * 16);
    L.k_words[0] = off; off = align256(off + U * L.tiles[0] * L.kw[0] * kTile * 4);
    L.k_meta[0] = off;  off = align256(off + U * L.kblocks * D * 4);
    L.sparse = off;     off = align256(off + U * (int64_t)c.capacity * c.sparse_per_vec * 4);
    L.v_words[0] = off; off = align256(off + U * L.vrows[0] * D * 4);
    L.v_meta[0] = off;  off = align256(off + U * L.tiles[0] * ng * kTile * 4);
    L.k_win = off;      off = align256(off + U * L.win_cap * D * 2);
    L.v_win = off;      off = align256(off + U * L.win_cap * D * 2);
  } else {
    return KVQ_ERR_ARG;
  }
  L.total_bytes = off;
  *out = L;
  return KVQ_OK;
}

extern "C" size_t kvq_workspace_bytes(const kvq_layout* lay, int32_t op, int32_t max_len) {
  if (!lay || max_len < 1 || max_len > lay->cfg.capacity) return 0;
  if (op == KVQ_OP_QUANTIZE) return quant_ws_plan(lay, max_len).total;
  if (op == KVQ_OP_DECODE) return decode_ws_bytes(lay, max_len, false);
  if (op == KVQ_OP_DECODE_MASS)
    return lay->cfg.mode == KVQ_MODE_TIERED ? decode_ws_bytes(lay, max_len, true) : 0;
  return 0;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" kvq_status kvq_set_channel_order(const kvq_layout* lay, void* cache, const int32_t* order,
                                            void* stream) {
  if (!lay || !cache || !order || !aligned16(cache)) return KVQ_ERR_ARG;
  const kvq_config& c = lay->cfg;
  if (c.mode != KVQ_MODE_TIERED || !c.reorder) return KVQ_ERR_UNSUPPORTED;
  for (int r = 0; r < 2 * c.kv_heads; ++r) {
    bool seen[kD] = {};
    for (int p = 0; p < kD; ++p) {
      const int32_t ch = order[(size_t)r * kD + p];
      if (ch < 0 || ch >= kD || seen[ch]) return KVQ_ERR_ARG;
      seen[ch] = true;
    }
  }
  uint8_t* base = (uint8_t*)cache + lay->chan_order;
  for (int h = 0; h < c.kv_heads; ++h) {
    uint8_t kb[kD], vb[kD];
    for (int p = 0; p < kD; ++p) {
      kb[p] = (uint8_t)order[(size_t)h * kD + p];
      vb[p] = (uint8_t)order[((size_t)c.kv_heads + h) * kD + p];
    }
    if (!launch_write_order(base + (size_t)h * kD, base + ((size_t)c.kv_heads + h) * kD, kb, vb, stream))
      return KVQ_ERR_LAUNCH;
  }
  return KVQ_OK;
}

extern "C" kvq_status kvq_quantize(const kvq_layout* lay, void* cache, const void* k, const void* v,
                                   int64_t stride_b, int64_t stride_t, int64_t stride_h,
                                   const float* scores, int32_t T, int32_t n_hi, int32_t* ranks_out,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (!lay || !cache || !k || !v) return KVQ_ERR_ARG;
  if (!aligned16(cache) || !aligned16(k) || !aligned16(v)) return KVQ_ERR_ARG;
  const kvq_config& c = lay->cfg;
  if (T < 1) return KVQ_ERR_ARG;
  if (T > c.capacity) return KVQ_ERR_CAPACITY;
  if (stride_b < 0 || stride_t < 0 || stride_h < 0) return KVQ_ERR_ARG;
  if ((stride_b | stride_t | stride_h) & 7) return KVQ_ERR_ARG;
  if (c.mode == KVQ_MODE_TIERED) {
    if (!scores || !aligned16(scores)) return KVQ_ERR_ARG;
    if (ranks_out && !aligned16(ranks_out)) return KVQ_ERR_ARG;
    if (n_hi < 0 || n_hi > T) return KVQ_ERR_ARG;
    if (n_hi > lay->cap[0] || T - n_hi > lay->cap[1]) return KVQ_ERR_CAPACITY;
    if (T > kMaxSortLen) return KVQ_ERR_UNSUPPORTED;
    QuantWs plan = quant_ws_plan(lay, T);
    if (!ws || !aligned16(ws) || ws_bytes < plan.total) return KVQ_ERR_WORKSPACE;
    if (!launch_rank_tiers(lay, (uint8_t*)cache, scores, T, n_hi, ranks_out, (uint8_t*)ws, plan, stream))
      return KVQ_ERR_LAUNCH;
    if (!launch_quantize_tiered(lay, (uint8_t*)cache, k, v, stride_b, stride_t, stride_h, T, n_hi,
                                (const uint8_t*)ws, plan, stream))
      return KVQ_ERR_LAUNCH;
    return KVQ_OK;
  }
  if (!launch_quantize_kchan(lay, (uint8_t*)cache, k, v, stride_b, stride_t, stride_h, T, stream))
    return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

extern "C" kvq_status kvq_append(const kvq_layout* lay, void* cache, const void* k_new,
                                 const void* v_new, const float* score_new, void* stream) {
  if (!lay || !cache || !k_new || !v_new || !score_new) return KVQ_ERR_ARG;
  if (!aligned16(cache) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(score_new))
    return KVQ_ERR_ARG;
  if (lay->cfg.mode != KVQ_MODE_TIERED) return KVQ_ERR_UNSUPPORTED;
  if (!launch_append(lay, (uint8_t*)cache, k_new, v_new, score_new, stream)) return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

extern "C" kvq_status kvq_decode_attn(const kvq_layout* lay, const void* cache, const void* q,
                                      float softmax_scale, int32_t max_len, void* out, void* ws,
                                      size_t ws_bytes, void* stream) {
  if (!lay || !cache || !q || !out) return KVQ_ERR_ARG;
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out)) return KVQ_ERR_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return KVQ_ERR_ARG;
  if (max_len < 1) return KVQ_ERR_ARG;
  if (max_len > lay->cfg.capacity) return KVQ_ERR_CAPACITY;
  size_t need = kvq_workspace_bytes(lay, KVQ_OP_DECODE, max_len);
  if (!ws || !aligned16(ws) || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  return launch_decode(lay, (const uint8_t*)cache, q, softmax_scale, max_len, out, (uint8_t*)ws, stream);
}

extern "C" kvq_status kvq_decode_attn_noalloc(const kvq_layout* lay, const void* cache, const void* q,
                                              float softmax_scale, int32_t max_len, void* out,
                                              void* stream) {
  if (!lay || !cache || !q || !out) return KVQ_ERR_ARG;
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out)) return KVQ_ERR_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return KVQ_ERR_ARG;
  if (max_len < 1) return KVQ_ERR_ARG;
  if (max_len > lay->cfg.capacity) return KVQ_ERR_CAPACITY;
  return launch_decode_noalloc(lay, (const uint8_t*)cache, q, softmax_scale, max_len, out, stream);
}

extern "C" size_t kvq_multi_workspace_bytes(const kvq_layout* lay, int32_t n_queries,
                                            int32_t max_len) {
  if (!lay || n_queries < 1 || n_queries > 4096 || max_len < 1 || max_len > lay->cfg.capacity)
    return 0;
  if (lay->cfg.mode != KVQ_MODE_TIERED) return 0;
  return decode_mq_ws_bytes(lay, n_queries, max_len);
}

extern "C" kvq_status kvq_decode_attn_multi(const kvq_layout* lay, const void* cache, const void* q,
                                            int32_t n_queries, float softmax_scale, int32_t max_len,
                                            void* out, float* lse, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (!lay || !cache || !q || !out) return KVQ_ERR_ARG;
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out)) return KVQ_ERR_ARG;
  if (lse && ((uintptr_t)lse & 3u)) return KVQ_ERR_ARG;
  if (n_queries < 1 || n_queries > 4096) return KVQ_ERR_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return KVQ_ERR_ARG;
  if (max_len < 1) return KVQ_ERR_ARG;
  if (max_len > lay->cfg.capacity) return KVQ_ERR_CAPACITY;
  if (lay->cfg.mode != KVQ_MODE_TIERED || lay->cfg.rope_theta != 0.0f) return KVQ_ERR_UNSUPPORTED;
  size_t need = kvq_multi_workspace_bytes(lay, n_queries, max_len);
  if (!ws || !aligned16(ws) || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  return launch_decode_mq(lay, (const uint8_t*)cache, q, n_queries, softmax_scale, max_len, out, lse,
                          (uint8_t*)ws, stream);
}

extern "C" kvq_status kvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                                      void* stream) {
  if (!buf || !sink || !aligned16(buf) || ((uintptr_t)sink & 3u)) return KVQ_ERR_ARG;
  if (bytes == 0 || (bytes & 15) || n_workgroups < 1 || n_workgroups > 65536) return KVQ_ERR_ARG;
  if (!launch_stream_read(buf, bytes, sink, n_workgroups, stream)) return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

extern "C" kvq_status kvq_decode_attn_mass(const kvq_layout* lay, const void* cache, const void* q,
                                           float softmax_scale, int32_t max_len, void* out, float* mass,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (!lay || !cache || !q || !out || !mass) return KVQ_ERR_ARG;
  if (!aligned16(cache) || !aligned16(q) || !aligned16(out) || ((uintptr_t)mass & 3u)) return KVQ_ERR_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return KVQ_ERR_ARG;
  if (max_len < 1) return KVQ_ERR_ARG;
  if (max_len > lay->cfg.capacity) return KVQ_ERR_CAPACITY;
  if (lay->cfg.mode != KVQ_MODE_TIERED) return KVQ_ERR_UNSUPPORTED;
  size_t need = kvq_workspace_bytes(lay, KVQ_OP_DECODE_MASS, max_len);
  if (!ws || !aligned16(ws) || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  return launch_decode(lay, (const uint8_t*)cache, q, softmax_scale, max_len, out, (uint8_t*)ws, stream,
                       mass);
}
