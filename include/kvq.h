/*
 * kvq.h - C ABI of the semantic mixed-precision KV-cache library for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources cited by page title and section):
 *
 *  - SemKV: Semantic Mixed-Precision KV Cache Quantization Guided by the
 *    Quality Cliff for Long-Context LLM Inference (arXiv 2608.28911),
 *    Abstract.  Every token of the KV cache is kept; tokens are ranked by a
 *    per-token model-internal score and each one is stored on one of two
 *    adjacent fractional-bit affine grids ("code bits/value" = log2 of the
 *    number of levels L, e.g. 5 levels = 2.322 bits); quantization also runs
 *    at generation time as tokens are appended.
 *  - SKVQ: Sliding-window Key and Value Cache Quantization for Large Language
 *    Models (arXiv 2405.06219), Abstract.  The most recent window of tokens
 *    stays in high precision (here: fp16); 2-bit keys.
 *  - KVQuant (summary post, "techniques" paragraph).  Keys quantized per
 *    channel; per-vector dense-and-sparse split with the outliers of each
 *    vector stored sparsely.
 *
 * Two cache modes:
 *   KVQ_MODE_TIERED  per-token score ranking; the top n_hi tokens of each
 *                    sequence use L_hi levels, the rest L_lo levels; affine
 *                    groups of `group` values along head_dim with fp16
 *                    (scale, zero) for keys and values.
 *   KVQ_MODE_KCHAN   keys quantized per channel over blocks of k_block
 *                    tokens at k_levels, with the sparse_per_vec entries of
 *                    largest magnitude of every key vector kept as fp16
 *                    (channel, value) pairs; values per token in groups of
 *                    v_group at v_levels; the last tokens (a window of
 *                    `window` up to window + k_block - 1) kept in fp16.
 *
 * Quantizer (both modes, one group of values x_i, fp16):
 *   z = min x_i (IEEE total order, -0 < +0), m = max x_i,
 *   (with clip: z = fp16_rne(fp32(z) * clip), m = fp16_rne(fp32(m) * clip)),
 *   s = fp16_rne( fp32(m - z) / fp32(L - 1) ),
 *   c_i = clamp( rint_even( fp32(x_i - z) / fp32(s) ), 0, L - 1 ),  s == 0 -> c_i = 0,
 *   dequantized value z + c_i * s.
 * Packing: a 32-bit word holds n_L = max{n : L^n <= 2^32} codes as
 *   sum_j c_j * L^j (little-endian base-L digits, unused digits 0).  Key codes
 *   are packed along head_dim within one token ("row words", ceil(D/n_L) per
 *   token); value codes are packed along the slot axis within one channel
 *   ("column words", one word per n_L slots per channel).
 * Rank: stable descending order of the fp32 score (equal scores keep token
 *   order; -0 == +0).  Tier 0 ("hi") iff rank < n_hi.  The slot of a token is
 *   its index among same-tier tokens in token order.
 * Generation-time tier: the new token of a sequence takes the hi grid iff its
 *   score is strictly greater than the median of the scores already in the
 *   sequence (mean of the two middle values for an even count, in fp64).
 * Attention: out = softmax(softmax_scale * q . k^) v^ over every cached token
 *   of the sequence, query head hq reads KV head hq / (q_heads / kv_heads).
 *   kvq_decode_attn_multi does the same for a block of new query tokens (with
 *   each row's log-sum-exp); kvq_decode_attn_mass also returns, per cached
 *   token, its softmax weight summed over the query heads.
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device pointers, 16-byte aligned.  `stream` is
 *     a hipStream_t (NULL = the default stream).  Calls are asynchronous on
 *     that stream; the library never allocates, frees or synchronizes.
 *   - The caller owns every buffer.  Inputs are read-only.  The cache is one
 *     device buffer of kvq_layout.total_bytes, written by kvq_quantize and
 *     kvq_append (and, for its channel orders, kvq_set_channel_order), read
 *     by kvq_decode_attn, kvq_decode_attn_multi and kvq_decode_attn_mass.
 *   - Arguments are validated on the host before any launch; on error the
 *     call returns a nonzero kvq_status and launches nothing.  A failed
 *     launch returns KVQ_ERR_LAUNCH.  Faults inside kernels surface at the
 *     caller's next synchronization.
 *   - Inputs must be finite, and so must every group scale in fp16.  The
 *     decode kernels form fp16 products 2^6 p * s of a softmax weight p <= 1
 *     and a value scale s; quantize and append set bit 1 of the sequence's
 *     counters[b][3] when they store a value scale of 1024 or more, and the
 *     decode kernels then use s / 2^6 in that product (for that sequence
 *     only), so every finite scale is accepted.
 *   - Per-channel-key mode: the decode kernel forms fp16 4 q_d s_d from the
 *     query and each channel's key scale, so |q_d| * s_d must stay below
 *     16376.
 *   - head_dim must be 128; q_heads / kv_heads must be 4 (grouped-query
 *     attention with four query heads per KV head).
 *   - Calls on one cache must not overlap (the library keeps no locks).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_ARG = 1,          /* null / misaligned pointer, bad size or stride */
  KVQ_ERR_UNSUPPORTED = 2,  /* a configuration the kernels do not implement */
  KVQ_ERR_CAPACITY = 3,     /* more tokens than the cache was laid out for */
  KVQ_ERR_WORKSPACE = 4,    /* workspace missing or too small */
  KVQ_ERR_LAUNCH = 5        /* a kernel launch failed */
} kvq_status;

enum { KVQ_MODE_TIERED = 0, KVQ_MODE_KCHAN = 1 };
enum { KVQ_OP_QUANTIZE = 0, KVQ_OP_DECODE = 1, KVQ_OP_DECODE_MASS = 2 };

/* Caller-filled description of one cache (host memory, plain data). */
typedef struct kvq_config {
  int32_t mode;           /* KVQ_MODE_TIERED or KVQ_MODE_KCHAN */
  int32_t batch;          /* sequences B >= 1; B * kv_heads <= 65536 (else KVQ_ERR_UNSUPPORTED) */
  int32_t kv_heads;       /* Hkv >= 1 */
  int32_t q_heads;        /* Hq = 4 * Hkv */
  int32_t head_dim;       /* D = 128 */
  int32_t capacity;       /* max tokens per sequence, <= 2^24 (else KVQ_ERR_UNSUPPORTED) */
  /* tiered mode */
  int32_t levels_hi;      /* L_hi in [3, 8]: the decode kernels expand digits through */
  int32_t levels_lo;      /* L_lo in [3, 8]   per-level tables (else KVQ_ERR_UNSUPPORTED) */
  int32_t group;          /* 32, 64 or 128 values per (scale, zero) */
  int32_t cap_hi;         /* slots reserved per hi pool (0 -> capacity) */
  int32_t cap_lo;         /* slots reserved per lo pool (0 -> capacity) */
  /* kchan mode */
  int32_t k_levels;       /* key levels in [3, 16] */
  int32_t k_block;        /* tokens per per-channel key group: 128 */
  int32_t v_levels;       /* value levels in [3, 16] */
  int32_t v_group;        /* values per value group: 32, 64 or 128 */
  int32_t window;         /* fp16 recent window, >= 0 */
  int32_t sparse_per_vec; /* fp16 outliers per key vector, 0..8 */
  /* tiered mode, optional (SKVQ, Abstract: channels rearranged so that each
   * quantization group holds alike channels; clipped group ranges) */
  int32_t reorder;        /* 1: stored channel orders (kvq_set_channel_order); 0: none */
  float clip;             /* 0: none; else in (0, 1]: group min and max scaled by clip */
  /* tiered mode, optional (KVQuant summary, "techniques": pre-RoPE key
   * quantization): keys are stored as given, before the rotary embedding,
   * and kvq_decode_attn / kvq_decode_attn_mass turn each dequantized key by
   * its token position: channel pair (2i, 2i + 1) by the angle
   * position * rope_theta^(-2i/128).  The query is passed already rotated.
   * A token's position is its index in the sequence (appended tokens
   * continue it).  Not with reorder = 1. */
  float rope_theta;       /* 0: none; else > 1: the rotary base (10000, 500000, ...) */
} kvq_config;

/* Filled by kvq_layout_init.  All offsets are bytes from the cache base;
 * index formulas below use element (not byte) units of the named type.
 *
 * unit u = b * kv_heads + h.  Tiered pools p = 0 (hi), 1 (lo).
 *
 *   counters  int32 [B][4]  = { length, n_hi, n_lo, flags } (kchan: { length,
 *             n_q, fp16 window tokens, flags }); flags bit 0: an append
 *             found its pool full; bit 1: a value scale >= 1024 is stored
 *   tokmap    uint32 [B][capacity]: slot | tier << 31 (tokens < length)
 *   sorted    float [B][capacity]: scores present, ascending (first length)
 *   key words (uint32) of slot s in pool p, word w < kw[p]:
 *       k_words[p] + (((u * tiles[p] + s/16) * kw[p] + w) * 16 + s%16)
 *   key / value (scale, zero) of slot s, group g < D/group, one uint32 with
 *   the fp16 scale in bits 0..15 and the fp16 zero in bits 16..31:
 *       k_meta[p] / v_meta[p] + (((u * tiles[p] + s/16) * (D/group) + g) * 16 + s%16)
 *   value words (uint32), slot s at digit s % nv[p] of row r = s / nv[p]:
 *       v_words[p] + ((u * vrows[p] + r) * D + d)
 *   with rope_theta > 0, slot positions int32 of slot s of pool p of sequence b:
 *       slot_pos[p] + (b * cap[p] + s) = the token index the slot holds
 *   with reorder = 1, channel orders uint8 [2][kv_heads][D] (keys, values):
 *       chan_order + (kv * kv_heads + h) * D + p = the channel whose code,
 *       like every index d above, sits at position p (groups are runs of
 *       `group` positions)
 *
 * kchan mode (slots are token indices t < n_q, n_q = k_block *
 * floor((T - window) / k_block)):
 *   key words:        k_words[0] + (((u * tiles[0] + t/16) * kw[0] + w) * 16 + t%16)
 *   key (scale,zero): k_meta[0] + ((u * kblocks + t / k_block) * D + d)
 *   sparse entries:   sparse + (u * capacity + t) * sparse_per_vec + e, each
 *                     uint32 channel << 16 | fp16 bits, channels ascending
 *   value words:      v_words[0] + ((u * vrows[0] + t / nv[0]) * D + d)
 *   value (scale,zero): v_meta[0] as in tiered mode with group = v_group
 *   fp16 window:      k_win / v_win + (u * win_cap + i) * D + d, i < T - n_q
 */
typedef struct kvq_layout {
  kvq_config cfg;
  int32_t nv[2];          /* codes per word: [0] hi / keys, [1] lo / values */
  int32_t kw[2];          /* key words per row per pool (kchan: kw[0]) */
  int32_t cap[2];         /* slots per pool (kchan: cap[0] = capacity) */
  int32_t tiles[2];       /* ceil(cap / 16) */
  int32_t vrows[2];       /* value word rows per unit and pool */
  int32_t kblocks;        /* kchan: per-channel key blocks per unit */
  int32_t win_cap;        /* kchan: fp16 window rows per unit */
  int32_t vnv;            /* kchan: value codes per word */
  int32_t reserved;
  int64_t counters, tokmap, sorted;
  int64_t k_words[2], k_meta[2], v_words[2], v_meta[2];
  int64_t sparse, k_win, v_win;
  int64_t chan_order;     /* tiered with reorder = 1; else 0 */
  int64_t slot_pos[2];    /* tiered with rope_theta > 0: int32 [B][cap[p]] token position of each slot; else 0 */
  int64_t total_bytes;
} kvq_layout;

/* Host only, pure.  Validates cfg and fills *out.  Returns KVQ_ERR_ARG /
 * KVQ_ERR_UNSUPPORTED for configurations outside the documented ranges. */
kvq_status kvq_layout_init(const kvq_config* cfg, kvq_layout* out);

/* Host only, pure.  Workspace bytes an operation needs for sequences of at
 * most max_len tokens (op = KVQ_OP_QUANTIZE or KVQ_OP_DECODE).  0 on bad
 * arguments. */
size_t kvq_workspace_bytes(const kvq_layout* lay, int32_t op, int32_t max_len);

/* Static string for a status code. */
const char* kvq_status_str(kvq_status s);

/* Stores the channel orders of a cache laid out with reorder = 1 (SKVQ,
 * Abstract: the channels of the KV cache are rearranged so that the channels
 * of each quantization group are alike; the order itself is calibrated
 * offline by the caller).  Call it before kvq_quantize / kvq_append; the
 * order is then used by every call on the cache: quantize and append read
 * channel order[p] into position p, decode reads q through the key order and
 * writes output channel order[p] from position p of the value sums.
 *   order:  HOST int32 [2][kv_heads][D]: [0] keys, [1] values; every row a
 *           permutation of 0..D-1 (else KVQ_ERR_ARG, nothing launched).
 *   One small launch per KV head on `stream` carries the bytes as kernel
 *   arguments; `order` may be reused as soon as the call returns.
 * KVQ_ERR_UNSUPPORTED if the cache was laid out with reorder = 0.  Without
 * this call such a cache gives undefined results (every access still stays
 * inside the cache and the caller's buffers). */
kvq_status kvq_set_channel_order(const kvq_layout* lay, void* cache, const int32_t* order,
                                 void* stream);

/* Quantize-on-write of a whole prefix (SemKV Abstract: rank, two adjacent
 * grids, every token kept; KVQuant / SKVQ for kchan mode).
 *   cache:   device, kvq_layout.total_bytes, fully (re)written except for
 *            the channel orders stored by kvq_set_channel_order, which it reads.
 *   k, v:    device fp16, element (b, t, h, d) at b*stride_b + t*stride_t +
 *            h*stride_h + d (d contiguous; strides in elements, multiples of 8).
 *   scores:  device fp32 [B][T] (tiered; NULL in kchan mode).
 *   T:       tokens per sequence, 1 <= T <= capacity (tiered: n_hi <= cap_hi
 *            and T - n_hi <= cap_lo; T <= 262144, else KVQ_ERR_UNSUPPORTED).
 *   n_hi:    tokens per sequence on the hi grid (tiered), 0 <= n_hi <= T.
 *   ranks_out: device int32 [B][T] or NULL (tiered).
 *   ws:      device workspace of at least kvq_workspace_bytes(lay,
 *            KVQ_OP_QUANTIZE, T) bytes. */
kvq_status kvq_quantize(const kvq_layout* lay, void* cache,
                        const void* k, const void* v,
                        int64_t stride_b, int64_t stride_t, int64_t stride_h,
                        const float* scores, int32_t T, int32_t n_hi,
                        int32_t* ranks_out, void* ws, size_t ws_bytes,
                        void* stream);

/* Generation-time quantize-on-append of one token per sequence (SemKV
 * Abstract: generation-time quantization), tiered mode only.  For each
 * sequence: tier from the running median, quantize K and V of every KV head
 * on that grid, store at the tier's next slot, record the score.
 *   k_new, v_new: device fp16 [B][Hkv][D];  score_new: device fp32 [B].
 *   A sequence whose pool is full is left unchanged and bit 0 of its
 *   counters[b][3] is set (the host can read it back); other sequences
 *   proceed. */
kvq_status kvq_append(const kvq_layout* lay, void* cache,
                      const void* k_new, const void* v_new,
                      const float* score_new, void* stream);

/* Decode attention of one query token per sequence over the whole packed
 * cache (dequantize, q.k^, online softmax, p.v^ in one pass over the packed
 * words; context split into chunks merged by log-sum-exp).
 *   q:       device fp16 [B][Hq][D].
 *   max_len: upper bound of any sequence's length (grid sizing); lengths and
 *            pool sizes are read from the cache counters.
 *   out:     device fp16 [B][Hq][D] (round to nearest even of the fp32 result).
 *   ws:      device workspace >= kvq_workspace_bytes(lay, KVQ_OP_DECODE, max_len). */
kvq_status kvq_decode_attn(const kvq_layout* lay, const void* cache,
                           const void* q, float softmax_scale, int32_t max_len,
                           void* out, void* ws, size_t ws_bytes, void* stream);

/* Decode attention as kvq_decode_attn for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument; the chunk partials live in a fixed
 * device array of the library (16 MiB per GPU, held until the process ends).
 * The call allocates and frees nothing.  Same arguments, outputs and kernels
 * as kvq_decode_attn (results are identical).  Returns KVQ_ERR_WORKSPACE,
 * launching nothing, when the partials of this call (4 x 132 fp32 per chunk
 * of every (sequence, KV head); the chunk split depends on the device and on
 * max_len) exceed 16 MiB.  Calls on one GPU share the array: calls that
 * overlap on one GPU (different streams or host threads) race and give
 * undefined results; calls on different GPUs are independent. */
kvq_status kvq_decode_attn_noalloc(const kvq_layout* lay, const void* cache,
                                   const void* q, float softmax_scale, int32_t max_len,
                                   void* out, void* stream);

/* Decode attention as kvq_decode_attn, plus the attention mass of every
 * cached token: the softmax weight it receives, summed over the sequence's
 * query heads (SemKV, Abstract: tokens are ranked by a model-internal score;
 * this is a score the decode step itself can hand back for re-ranking).  The
 * masses of a sequence sum to Hq.  Tiered mode only.
 *   mass:  device fp32 [B][max_len]; entry (b, t) for token index t of
 *          sequence b (insertion order, appended tokens included), 0 past
 *          the sequence's length.
 *   ws:    device workspace >= kvq_workspace_bytes(lay, KVQ_OP_DECODE_MASS,
 *          max_len) (the partials, each pool's raw scores, per-head sums).
 * Returns KVQ_ERR_UNSUPPORTED for the per-channel-key mode. */
kvq_status kvq_decode_attn_mass(const kvq_layout* lay, const void* cache,
                                const void* q, float softmax_scale, int32_t max_len,
                                void* out, float* mass, void* ws, size_t ws_bytes,
                                void* stream);

/* Workspace bytes of kvq_decode_attn_multi for n_queries query tokens per
 * sequence and sequences of at most max_len tokens; 0 on bad arguments. */
size_t kvq_multi_workspace_bytes(const kvq_layout* lay, int32_t n_queries, int32_t max_len);

/* Attention of a block of new query tokens per sequence over the whole packed
 * cache: the quantized history read again when a conversation continues
 * (SemKV, Abstract: the cache reappears across turns).  Every query row reads
 * every cached token (no mask: the cache precedes the new tokens); rows are
 * independent.  Four query tokens share each expansion of the packed words
 * on the matrix cores.  Tiered mode only.
 *   q:         device fp16 [B][n_queries][Hq][D].
 *   n_queries: 1 .. 4096.
 *   out:       device fp16 [B][n_queries][Hq][D] (round to nearest even).
 *   lse:       device fp32 [B][n_queries][Hq] or NULL: ln sum_t exp(scale q.k^_t)
 *              of each row, for merging with attention over the new tokens.
 *   ws:        device workspace >= kvq_multi_workspace_bytes(lay, n_queries, max_len).
 * Returns KVQ_ERR_UNSUPPORTED for the per-channel-key mode and for caches
 * laid out with rope_theta > 0. */
kvq_status kvq_decode_attn_multi(const kvq_layout* lay, const void* cache,
                                 const void* q, int32_t n_queries, float softmax_scale,
                                 int32_t max_len, void* out, float* lse,
                                 void* ws, size_t ws_bytes, void* stream);

/* Measurement aid, not part of the method: reads every byte of a device
 * buffer once (16-byte loads, coalesced) to measure the achievable HBM read
 * bandwidth, the reference beside the published peak for the rates of the
 * entry points above.
 *   buf:   device pointer, 16-byte aligned; bytes: a multiple of 16, > 0.
 *   sink:  device uint32 [n_workgroups], written (the xor of what was read).
 *   n_workgroups: 1 .. 65536 (256 threads each).
 * KVQ_ERR_ARG on a null or misaligned pointer or a bad size. */
kvq_status kvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t n_workgroups,
                           void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
