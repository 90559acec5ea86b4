// Quantize-on-write (SemKV, Abstract: affine quantizer on an L-level
// fractional-bit grid, two adjacent grids chosen by rank, every token kept,
// also at generation time) and the per-channel-key / dense-and-sparse /
// fp16-window variant (KVQuant summary, "techniques"; SKVQ, Abstract).
//
// A workgroup owns a whole number of value word rows (nv slots each, at most
// 256 slots) of one pool of one (sequence, KV head), so every packed word it
// writes is complete.  Codes are staged in LDS as bytes,
// then packed twice: along head_dim for keys (row words) and along slots for
// values (column words).
#include <string.h>

#include "common.h"
#include "internal.h"
#include "digits.h"

namespace kvq {

constexpr int kQThreads = 256;

__host__ __device__ inline int rows_per_wg(int nv) { return nv >= 256 ? 1 : 256 / nv; }

struct QuantArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, st, sh;
  const int32_t* inv;      // [B][cap] slot -> token, or null for identity
  int inv_cap;
  int n;                   // valid slots per unit (same for every sequence)
  int L, nv, kw, tiles, vrows, Hkv;
  uint32_t* kwords;        // null: values only
  uint32_t* kmeta;
  uint32_t* vwords;
  uint32_t* vmeta;
  const uint8_t* korder = nullptr;   // [Hkv][128] stored key channel order, or null
  const uint8_t* vorder = nullptr;   // [Hkv][128] stored value channel order, or null
  float clip = 1.0f;                 // group min/max scale factor (1: none)
  int32_t* counters = nullptr;       // [B][4]: flags word 3 gets kFlagBigValueScale
};

// Quantize one group of G fp16 values at src (16-byte aligned); codes to LDS.
template <int G>
__device__ inline uint32_t quant_group(const uint16_t* __restrict__ src, int L, uint8_t* codes) {
  uint4 raw[G / 8];
#pragma unroll
  for (int i = 0; i < G / 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(src + i * 8);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(raw);
  int kmn = f16_order_key(x[0]), kmx = kmn;
#pragma unroll
  for (int i = 1; i < G; ++i) {
    int kk = f16_order_key(x[i]);
    kmn = min(kmn, kk);
    kmx = max(kmx, kk);
  }
  const uint32_t mn = f16_from_order_key(kmn), mx = f16_from_order_key(kmx);
  GroupQ g = group_setup(mn, mx, L);
#pragma unroll
  for (int i = 0; i < G; ++i) codes[i] = (uint8_t)quant_value(h2f(x[i]), g);
  return g.s_bits | (mn << 16);
}

template <int G>
__global__ __launch_bounds__(kQThreads) void k_quant_pool(QuantArgs a) {
  extern __shared__ uint8_t lds[];
  constexpr int NG = kD / G;
  const int rows = rows_per_wg(a.nv);
  const int SL = rows * a.nv;
  uint8_t* ck = lds;                 // [SL][128] key codes
  uint8_t* cv = lds + SL * kD;       // [SL][128] value codes
  const int tid = threadIdx.x;
  const int u = blockIdx.y;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int s0 = blockIdx.x * SL;
  const int kv_lo = a.kwords ? 0 : 1;
  // phase 1: groups -> codes (LDS) and (scale, zero) (global)
  const int ntask = SL * NG * 2;
  for (int task = tid; task < ntask; task += kQThreads) {
    const int kv = task / (SL * NG);
    if (kv < kv_lo) continue;
    const int rem = task - kv * SL * NG;
    const int i = rem / NG, g = rem - (rem / NG) * NG;
    const int s = s0 + i;
    uint8_t* dst = (kv ? cv : ck) + i * kD + g * G;
    uint32_t meta = 0;
    if (s < a.n) {
      const int t = a.inv ? a.inv[(size_t)b * a.inv_cap + s] : s;
      const uint16_t* src = (kv ? a.v : a.k) + b * a.sb + (int64_t)t * a.st + h * a.sh + g * G;
      meta = quant_group<G>(src, a.L, dst);
      if (kv && (meta & 0x7FFFu) >= kBigScaleBits) atomicOr(a.counters + b * 4 + 3, kFlagBigValueScale);
    } else {
#pragma unroll
      for (int i2 = 0; i2 < G; ++i2) dst[i2] = 0;
    }
    if (s < a.tiles * kTile) {
      uint32_t* mp = kv ? a.vmeta : a.kmeta;
      mp[(((size_t)u * a.tiles + s / kTile) * NG + g) * kTile + (s % kTile)] = meta;
    }
  }
  __syncthreads();
  // phase 2: key row words
  if (a.kwords) {
    for (int task = tid; task < SL * a.kw; task += kQThreads) {
      const int i = task / a.kw, w = task - (task / a.kw) * a.kw;
      const int s = s0 + i;
      if (s >= a.tiles * kTile) continue;
      const int d0 = w * a.nv;
      const int d1 = min(kD, d0 + a.nv);
      uint32_t word = 0;
      for (int d = d1 - 1; d >= d0; --d) word = word * (uint32_t)a.L + ck[i * kD + d];
      a.kwords[(((size_t)u * a.tiles + s / kTile) * a.kw + w) * kTile + (s % kTile)] = word;
    }
  }
  // phase 3: value column words (rows of nv slots)
  const int r0 = s0 / a.nv;
  for (int task = tid; task < rows * kD; task += kQThreads) {
    const int r = task / kD, d = task % kD;
    if (r0 + r >= a.vrows) continue;
    uint32_t word = 0;
    for (int j = a.nv - 1; j >= 0; --j) word = word * (uint32_t)a.L + cv[(r * a.nv + j) * kD + d];
    a.vwords[((size_t)u * a.vrows + r0 + r) * kD + d] = word;
  }
}

// ---- row kernel: four lanes per slot row (fast path, L <= 8) ----
//
// Four lanes (a quad) per slot row: load i of lane q reads channels
// 32 i + 8 q .. 32 i + 8 q + 7, so each load instruction covers 64
// contiguous bytes of sixteen rows and a group of G channels is chunks
// i in [G/32 g, G/32 (g + 1)) of all four lanes.  Group extremes use the
// IEEE-2019 minimum/maximum (-0 below +0) on packed fp16, with the maximum
// carried negated so that one packed minimum reduces both over the quad
// (DPP lane permutes).  Lane q then forms the fp16 scale/zero of one group
// (with the exact quotient of group_setup) and the quad shares them.  Codes
// go to LDS as bytes; key row words (along head_dim) and value column words
// (along slots) are packed from there in fp32 Horner halves (exact below
// 2^24) joined by one 24-bit integer multiply-add.
template <int L>
struct RowPack {
  static constexpr int NV = cpw(L);
  static constexpr int KW = (kD + NV - 1) / NV;
  static constexpr int ROWS = NV >= 256 ? 1 : 256 / NV;   // value word rows per workgroup
  static constexpr int SL = ROWS * NV;                    // slots per workgroup (<= 256)
  // Horner over chunks of CS digits: a chunk is one 4-byte dot product with
  // byte weights L^0 .. L^(CS-1) (each below 256)
  static constexpr int CS = ipow(L, 3) <= 255u ? 4 : 3;
  static constexpr int NCH = (NV + CS - 1) / CS;
  static constexpr uint32_t LCS = ipow(L, CS);
  // byte weights of a chunk whose first n digits count
  static constexpr uint32_t weights(int n) {
    uint32_t w = 0;
    for (int k = 0; k < CS && k < n; ++k) w |= ipow(L, k) << (8 * k);
    return w;
  }
  // acc * L^CS + p, exact: 24-bit multiply while the accumulator stays below
  // 2^24 (L^(digits above this chunk) bounds it)
  __device__ static inline uint32_t horner(uint32_t acc, uint32_t p, int above) {
    return ipow(L, above) <= (1u << 24) ? __umul24(acc, LCS) + p : acc * LCS + p;
  }
  // key word w of a code row (bytes = channels; entries past head_dim count 0)
  __device__ static inline uint32_t key_word(const uint32_t* row, int w) {
    uint32_t acc = 0;
#pragma unroll
    for (int k = NCH - 1; k >= 0; --k) {
      const int d0 = w * NV + CS * k;                     // first channel of the chunk
      const int n = min(min(CS, NV - CS * k), kD - d0);   // digits that count
      uint32_t p = 0;
      if (n > 0) {
        const int o = d0 >> 2, sh = d0 & 3;
        const uint32_t bytes = sh == 0 ? row[o] : __builtin_amdgcn_alignbyte(row[o + 1], row[o], sh);
        p = __builtin_amdgcn_udot4(bytes, weights(n), 0u, false);
      }
      acc = k == NCH - 1 ? p : horner(acc, p, NV - CS * (k + 1));
    }
    return acc;
  }
  // four value column words from NV code dwords (dword jj = slot jj of the
  // word row, byte c = channel c): 4x4 byte transposes feed the dot products
  __device__ static inline uint4 value_words(const uint32_t* col) {
    uint32_t acc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = NCH - 1; k >= 0; --k) {
      const int j0 = CS * k, n = min(CS, NV - j0);
      const uint32_t d0 = col[j0], d1 = n > 1 ? col[j0 + 1] : 0u;
      const uint32_t d2 = n > 2 ? col[j0 + 2] : 0u, d3 = n > 3 ? col[j0 + 3] : 0u;
      const uint32_t lo01 = __builtin_amdgcn_perm(d1, d0, 0x05010400u);
      const uint32_t hi01 = __builtin_amdgcn_perm(d1, d0, 0x07030602u);
      const uint32_t lo23 = __builtin_amdgcn_perm(d3, d2, 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(d3, d2, 0x07030602u);
      const uint32_t t[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                             __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                             __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                             __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t p = __builtin_amdgcn_udot4(t[c], weights(n), 0u, false);
        acc[c] = k == NCH - 1 ? p : horner(acc[c], p, NV - CS * (k + 1));
      }
    }
    return make_uint4(acc[0], acc[1], acc[2], acc[3]);
  }
};

__device__ inline h2v hb(uint32_t x) { return h2_from_bits(x); }
__device__ inline uint32_t bh(h2v x) { return __builtin_bit_cast(uint32_t, x); }
// packed fp16 IEEE-2019 minimum / maximum
__device__ inline uint32_t hmin(uint32_t x, uint32_t y) { return bh(__builtin_elementwise_minimum(hb(x), hb(y))); }
__device__ inline uint32_t hmax(uint32_t x, uint32_t y) { return bh(__builtin_elementwise_maximum(hb(x), hb(y))); }
// value of another lane of the same 16-lane row via a DPP move: a quad
// permute (CTRL < 0x100) or a row pattern such as the mirrors below
template <int CTRL>
__device__ inline uint32_t quad_perm(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;    // quad_perm [1,0,3,2], [2,3,0,1]
constexpr int kRowHalfMirror = 0x141, kRowMirror = 0x140;   // lane i <-> 7 - i (per 8), 15 - i
template <int O>
__device__ inline uint32_t quad_bcast(uint32_t v) { return quad_perm<O * 0x55>(v); }

// q = RN(fl32(x - z) / s) by the quotient correction of group_setup (s == 0
// gives r = 0 and q = 0); z and s are the fp16 halves of the meta word.
// `one` is 1.0 hidden from the optimizer so that x * one - z stays a single
// mixed-precision fma on the fp16 input.
__device__ inline float quotient_of(_Float16 x, _Float16 z, _Float16 s, float r, float one) {
  const float a = __builtin_fmaf((float)x, one, -(float)z);    // fl32(x - z), one rounding
  const float q0 = a * r;
  const float rho = __builtin_fmaf(-q0, (float)s, a);
  return __builtin_fmaf(rho, r, q0);
}

// (min, -max) of the 8 CPG fp16 values of a lane's chunks of one group
template <int CPG>
__device__ inline uint32_t chunk_extremes(const uint4* x) {
  uint32_t lo = x[0].x, hi = x[0].x;
#pragma unroll
  for (int c = 0; c < CPG; ++c) {
    const uint32_t w[4] = {x[c].x, x[c].y, x[c].z, x[c].w};
#pragma unroll
    for (int j = (c == 0 ? 1 : 0); j < 4; ++j) {
      lo = hmin(lo, w[j]);
      hi = hmax(hi, w[j]);
    }
  }
  // halves side by side: (lo.lo, -hi.lo) and (lo.hi, -hi.hi)
  const uint32_t e0 = __builtin_amdgcn_perm(hi, lo, 0x05040100u) ^ 0x80000000u;
  const uint32_t e1 = __builtin_amdgcn_perm(hi, lo, 0x07060302u) ^ 0x80000000u;
  return hmin(e0, e1);
}

// codes of the 8 values of one chunk (fp16 bits in x) into two byte words;
// CLAMP bounds the quotient by the top level (needed only for subnormal
// scales, where s can be far below range / (L - 1)); LOW bounds it below by 0
// (clipped ranges, where values can lie below the zero point)
template <int L, bool CLAMP, bool LOW = false>
__device__ inline void chunk_codes(uint4 x, uint32_t meta, float r, float one, uint32_t& c0, uint32_t& c1) {
  const h2v zs = hb(meta);                    // (s, z)
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float q = quotient_of(hb(w[e / 2])[e & 1], zs[1], zs[0], r, one);
    if (LOW) q = fmaxf(q, 0.0f);
    if (CLAMP) q = fminf(q, (float)(L - 1));
    c[e / 4] = __builtin_amdgcn_cvt_pk_u8_f32(q, e & 3, c[e / 4]);
  }
  c0 = c[0];
  c1 = c[1];
}

// Orders the LDS accesses of one wave (stores before the loads that follow);
// the wave's own LDS operations complete in issue order.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Clipped group range: min and max each scaled by clip in fp32, then rounded
// to fp16 (two roundings, kept apart from any fused form).
__device__ inline void clip_range(uint32_t& mn, uint32_t& mx, float clip) {
  float lo = h2f(mn) * clip, hi = h2f(mx) * clip;
  asm volatile("" : "+v"(lo), "+v"(hi));
  mn = f2h_rne(lo);
  mx = f2h_rne(hi);
}

// SKVQ selects the variant with stored channel orders and clipped group
// ranges: each wave's rows go through LDS (natural order in, 8-byte stores)
// and come back gathered in the stored order, so the rest of the kernel sees
// stored positions; codes are then bounded at both ends.
template <int L, int G, bool SKVQ>
__global__ __launch_bounds__(kQThreads) void k_quant_rows(QuantArgs a) {
  using P = RowPack<L>;
  constexpr int NV = P::NV, KW = P::KW, NG = kD / G, SL = P::SL, ROWS = P::ROWS;
  constexpr int NP = (SL + 31) / 32;               // rows per thread (32 rows per pass)
  constexpr int CW = kD / 4 + 1;                   // dwords per code row (+1: bank spread)
  static_assert(NG >= 1 && NG <= 4, "group of 32, 64 or 128 channels");
  __shared__ uint32_t codes[SL][CW];               // byte codes, [slot][channel]
  __shared__ int tok[256];
  constexpr int SW = kD / 2 + 2;                   // dwords per staged fp16 row (+2: bank spread)
  __shared__ uint32_t stage[SKVQ ? 64 : 1][SW];    // one pass of rows, natural channel order
  const int tid = threadIdx.x, u = blockIdx.y;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int s0 = blockIdx.x * SL;
  // eight lanes per row: lane q holds channels 64 i + 8 q .. 64 i + 8 q + 7
  // (i = 0, 1), so one load instruction reads whole 128-byte lines of eight
  // rows; a 32-channel group is one quad of the eight
  const int q = tid & 7, rp = tid >> 3;            // lane in the row's eight, row of the pass
  const int qh = q >> 2, ql = q & 3;               // quad of the row, lane in the quad
  {
    const int s = s0 + tid;
    tok[tid] = (tid < SL && s < a.n) ? (a.inv ? a.inv[(size_t)b * a.inv_cap + s] : s) : -1;
  }
  __syncthreads();
  float one = 1.0f;
  asm volatile("" : "+v"(one));
  const int tiled = a.tiles * kTile;
  // the group whose scale this lane forms (two lanes per group for G 32,
  // four for G 64, all eight for G 128), and whether it writes its (scale, zero)
  const int gown = G == 32 ? 2 * (ql & 1) + qh : G == 64 ? (ql & 1) : 0;
  const bool owner = G == 32 ? ql < 2 : q < NG;
  for (int kv = a.kwords ? 0 : 1; kv < 2; ++kv) {
    const uint16_t* base = (kv ? a.v : a.k) + b * a.sb + h * a.sh + 8 * q;
    uint4 x[NP][2];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = tok[rp + 32 * p];              // -1: no token (values 0, codes 0)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        x[p][i] = t >= 0 ? ld_stream16(base + (int64_t)t * a.st + 64 * i) : make_uint4(0u, 0u, 0u, 0u);
    }
    // stored channel orders: bytes of the channels at positions
    // 64 i + 8 q .. 64 i + 8 q + 7 of this lane
    const uint8_t* ord = SKVQ ? (kv ? a.vorder : a.korder) : nullptr;
    uint32_t ow[4];
    if (SKVQ && ord) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          ow[2 * i + j] = *reinterpret_cast<const uint32_t*>(ord + (size_t)h * kD + 64 * i + 8 * q + 4 * j);
    }
    if (SKVQ && ord) {
      // every pass's rows through LDS, gathered back in the stored order; a
      // wave stages and gathers only its own 8 rows, so a wave-level
      // barrier orders its accesses (no workgroup barrier)
      uint32_t* srow = stage[rp];
      const uint16_t* hrow = reinterpret_cast<const uint16_t*>(srow);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        wave_lds_sync();                             // the previous pass has been gathered
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          *reinterpret_cast<uint2*>(srow + 32 * i + 4 * q) = make_uint2(x[p][i].x, x[p][i].y);
          *reinterpret_cast<uint2*>(srow + 32 * i + 4 * q + 2) = make_uint2(x[p][i].z, x[p][i].w);
        }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const uint32_t ob = ow[2 * i + e / 4];
            const uint32_t c0 = (ob >> (8 * (e % 4))) & 0x7Fu, c1 = (ob >> (8 * (e % 4) + 8)) & 0x7Fu;
            w[e / 2] = (uint32_t)hrow[c0] | ((uint32_t)hrow[c1] << 16);
          }
          x[p][i] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
    }
    uint32_t* mp = kv ? a.vmeta : a.kmeta;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = rp + 32 * p;
      // extremes of each load's chunk over its quad (G 32), over the row's
      // eight lanes (G 64: the two quads through the half-row mirror), and
      // over both loads as well (G 128); lane q keeps group gown
      uint32_t e[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t v = chunk_extremes<1>(&x[p][i]);
        v = hmin(v, quad_perm<kQuadXor1>(v));
        v = hmin(v, quad_perm<kQuadXor2>(v));
        if (G >= 64) v = hmin(v, quad_perm<kRowHalfMirror>(v));
        e[i] = v;
      }
      const uint32_t eo = G == 128 ? hmin(e[0], e[1]) : e[ql & 1];
      uint32_t mn = eo & 0xFFFFu, mx = (eo >> 16) ^ 0x8000u;
      if constexpr (SKVQ) clip_range(mn, mx, a.clip);
      GroupQ gq = group_setup(mn, mx, L);
      if (gq.s == 0.0f) gq.r = 0.0f;               // all codes 0
      if (kv) flag_big_value_scale(a.counters, b, gq.s_bits);
      const uint32_t meta = gq.s_bits | (mn << 16);
      const bool sub = (gq.s_bits & 0x7C00u) == 0u;    // zero or subnormal scale
      if (r < SL && owner) {
        const int s = s0 + r;
        if (s < tiled) mp[(((size_t)u * a.tiles + s / kTile) * NG + gown) * kTile + (s % kTile)] = meta;
      }
      // each load's (meta, r) from its group's owner in the quad: lane i of
      // the quad forms the group of load i (G 32 and 64); G 128 has one group
      uint32_t gm[2], gr[2];
      if (G == 128) {
        gm[0] = gm[1] = meta;
        gr[0] = gr[1] = __float_as_uint(gq.r);
      } else {
        gm[0] = quad_bcast<0>(meta);
        gr[0] = quad_bcast<0>(__float_as_uint(gq.r));
        gm[1] = quad_bcast<1>(meta);
        gr[1] = quad_bcast<1>(__float_as_uint(gq.r));
      }
      uint32_t c[2][2];
      if constexpr (SKVQ) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          chunk_codes<L, true, true>(x[p][i], gm[i], __uint_as_float(gr[i]), one, c[i][0], c[i][1]);
      } else if (__builtin_expect(__ballot(sub && gq.s != 0.0f) != 0ull, 0)) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          chunk_codes<L, true>(x[p][i], gm[i], __uint_as_float(gr[i]), one, c[i][0], c[i][1]);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          chunk_codes<L, false>(x[p][i], gm[i], __uint_as_float(gr[i]), one, c[i][0], c[i][1]);
      }
      if (r < SL) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          codes[r][16 * i + 2 * q] = c[i][0];
          codes[r][16 * i + 2 * q + 1] = c[i][1];
        }
      }
    }
    __syncthreads();
    if (kv == 0) {
      // key row words: one slot per thread, its code row read once
      if (tid < SL && s0 + tid < tiled) {
        const int s = s0 + tid;
        uint32_t row[CW];
#pragma unroll
        for (int j = 0; j < CW; ++j) row[j] = codes[tid][j];
        uint32_t* dst = a.kwords + (((size_t)u * a.tiles + s / kTile) * KW) * kTile + (s % kTile);
#pragma unroll
        for (int w = 0; w < KW; ++w) dst[w * kTile] = P::key_word(row, w);
      }
    } else {
      // value column words: task (word row rr, channels 4 d4 .. 4 d4 + 3)
      const int r0 = s0 / NV;
      for (int task = tid; task < ROWS * (kD / 4); task += kQThreads) {
        const int rr = task / (kD / 4), d4 = task % (kD / 4);
        if (r0 + rr >= a.vrows) continue;
        uint32_t col[NV];
#pragma unroll
        for (int jj = 0; jj < NV; ++jj) col[jj] = codes[rr * NV + jj][d4];
        *reinterpret_cast<uint4*>(&a.vwords[((size_t)u * a.vrows + r0 + rr) * kD + 4 * d4]) =
            P::value_words(col);
      }
    }
    __syncthreads();
  }
}

template <int L, bool SKVQ>
static bool launch_rows_LS(const QuantArgs& a, int G, dim3 grid, hipStream_t s) {
  switch (G) {
    case 32: k_quant_rows<L, 32, SKVQ><<<grid, kQThreads, 0, s>>>(a); return true;
    case 64: k_quant_rows<L, 64, SKVQ><<<grid, kQThreads, 0, s>>>(a); return true;
    case 128: k_quant_rows<L, 128, SKVQ><<<grid, kQThreads, 0, s>>>(a); return true;
  }
  return false;
}

template <int L>
static bool launch_rows_L(const QuantArgs& a, int G, dim3 grid, hipStream_t s) {
  const bool skvq = a.korder || a.vorder || a.clip != 1.0f;
  return skvq ? launch_rows_LS<L, true>(a, G, grid, s) : launch_rows_LS<L, false>(a, G, grid, s);
}

static bool launch_pool(const QuantArgs& a, int G, int U, hipStream_t s) {
  const int SL = rows_per_wg(a.nv) * a.nv;
  const int cover = max(a.tiles * kTile, a.vrows * a.nv);
  dim3 grid(ceil_div(cover, SL), U);
  switch (a.L) {
    case 3: return launch_rows_L<3>(a, G, grid, s);
    case 4: return launch_rows_L<4>(a, G, grid, s);
    case 5: return launch_rows_L<5>(a, G, grid, s);
    case 6: return launch_rows_L<6>(a, G, grid, s);
    case 7: return launch_rows_L<7>(a, G, grid, s);
    case 8: return launch_rows_L<8>(a, G, grid, s);
  }
  if (a.korder || a.vorder || a.clip != 1.0f) return false;   // the row kernel covers L <= 8 only
  size_t lds = (size_t)2 * SL * kD;
  switch (G) {
    case 32: k_quant_pool<32><<<grid, kQThreads, lds, s>>>(a); break;
    case 64: k_quant_pool<64><<<grid, kQThreads, lds, s>>>(a); break;
    case 128: k_quant_pool<128><<<grid, kQThreads, lds, s>>>(a); break;
    default: return false;
  }
  return true;
}

bool launch_quantize_tiered(const kvq_layout* L, uint8_t* cache, const void* k, const void* v,
                            int64_t sb, int64_t st, int64_t sh, int T, int n_hi,
                            const uint8_t* ws, const QuantWs& plan, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int U = L->cfg.batch * L->cfg.kv_heads;
  const int lv[2] = {L->cfg.levels_hi, L->cfg.levels_lo};
  const int np[2] = {n_hi, T - n_hi};
  for (int p = 0; p < 2; ++p) {
    QuantArgs a;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.sb = sb; a.st = st; a.sh = sh;
    a.inv = (const int32_t*)(ws + plan.inv[p]);
    a.inv_cap = L->cap[p];
    a.n = np[p];
    a.L = lv[p]; a.nv = L->nv[p]; a.kw = L->kw[p]; a.tiles = L->tiles[p]; a.vrows = L->vrows[p];
    a.Hkv = L->cfg.kv_heads;
    a.kwords = (uint32_t*)(cache + L->k_words[p]);
    a.kmeta = (uint32_t*)(cache + L->k_meta[p]);
    a.vwords = (uint32_t*)(cache + L->v_words[p]);
    a.vmeta = (uint32_t*)(cache + L->v_meta[p]);
    a.korder = L->cfg.reorder ? cache + L->chan_order : nullptr;
    a.vorder = L->cfg.reorder ? cache + L->chan_order + (size_t)L->cfg.kv_heads * kD : nullptr;
    a.clip = L->cfg.clip > 0.0f ? L->cfg.clip : 1.0f;
    a.counters = (int32_t*)(cache + L->counters);
    if (!launch_pool(a, L->cfg.group, U, s)) return false;
  }
  return hipGetLastError() == hipSuccess;
}

// ---------------------------------------------------------------- kchan ----
// One workgroup per (unit, 128-token key block): per key vector pick the
// sparse_per_vec largest |x| (ties -> lower channel) into the sparse list and
// zero them; per channel quantize the dense block (min/max over 128 tokens);
// pack each token's codes along head_dim.
__global__ __launch_bounds__(256) void k_kchan_keys(const uint16_t* __restrict__ k, int64_t sb,
                                                    int64_t st, int64_t sh, int Hkv, int L,
                                                    int nv, int kw, int tiles, int kblocks,
                                                    int cap, int spv,
                                                    uint32_t* __restrict__ kwords,
                                                    uint32_t* __restrict__ kmeta,
                                                    uint32_t* __restrict__ sparse) {
  __shared__ uint16_t xs[128][kD + 2];     // dense block, padded rows
  __shared__ uint8_t cs[128][kD];          // codes
  const int tid = threadIdx.x;
  const int blk = blockIdx.x, u = blockIdx.y;
  const int b = u / Hkv, h = u % Hkv;
  const int t0 = blk * 128;
  for (int e = tid; e < 128 * kD / 8; e += 256) {
    const int t = e / (kD / 8), c8 = (e % (kD / 8)) * 8;
    uint4 raw = *reinterpret_cast<const uint4*>(k + b * sb + (int64_t)(t0 + t) * st + h * sh + c8);
    const uint16_t* r = reinterpret_cast<const uint16_t*>(&raw);
    for (int i = 0; i < 8; ++i) xs[t][c8 + i] = r[i];
  }
  __syncthreads();
  if (tid < 128) {
    const int t = tid;
    int chosen[8];
    for (int e = 0; e < spv; ++e) {
      int best = -1;
      uint32_t bmag = 0;
      for (int d = 0; d < kD; ++d) {
        bool taken = false;
        for (int e2 = 0; e2 < e; ++e2) taken |= (chosen[e2] == d);
        const uint32_t m = xs[t][d] & 0x7FFFu;
        if (!taken && (best < 0 || m > bmag)) { best = d; bmag = m; }
      }
      chosen[e] = best;
    }
    // ascending channel order
    for (int i = 1; i < spv; ++i)
      for (int j = i; j > 0 && chosen[j - 1] > chosen[j]; --j) {
        int x = chosen[j]; chosen[j] = chosen[j - 1]; chosen[j - 1] = x;
      }
    // each thread owns its token row: read the outliers, then zero them
    for (int e = 0; e < spv; ++e) {
      const uint32_t ent = ((uint32_t)chosen[e] << 16) | xs[t][chosen[e]];
      sparse[((size_t)u * cap + t0 + t) * spv + e] = ent;
    }
    for (int e = 0; e < spv; ++e) xs[t][chosen[e]] = 0;
  }
  __syncthreads();
  if (tid < kD) {
    const int d = tid;
    int kmn = f16_order_key(xs[0][d]), kmx = kmn;
    for (int t = 1; t < 128; ++t) {
      int kk = f16_order_key(xs[t][d]);
      kmn = min(kmn, kk);
      kmx = max(kmx, kk);
    }
    const uint32_t mn = f16_from_order_key(kmn), mx = f16_from_order_key(kmx);
    GroupQ g = group_setup(mn, mx, L);
    for (int t = 0; t < 128; ++t) cs[t][d] = (uint8_t)quant_value(h2f(xs[t][d]), g);
    kmeta[((size_t)u * kblocks + blk) * kD + d] = g.s_bits | (mn << 16);
  }
  __syncthreads();
  for (int task = tid; task < 128 * kw; task += 256) {
    const int t = task / kw, w = task % kw;
    const int s = t0 + t;
    const int d0 = w * nv, d1 = min(kD, d0 + nv);
    uint32_t word = 0;
    for (int d = d1 - 1; d >= d0; --d) word = word * (uint32_t)L + cs[t][d];
    kwords[(((size_t)u * tiles + s / kTile) * kw + w) * kTile + (s % kTile)] = word;
  }
}

// Data-parallel form of the same block step for grids of 3..8 levels and at
// most two sparse entries per key vector.  Sixteen lanes per token row (eight
// channels each, eight rows per lane): the row's largest magnitudes come from
// a 16-lane DPP exchange over keys (|x| bits << 16 | 0xFFFF - channel, so ties
// go to the lower channel); the owning lane writes each sparse entry and
// zeroes it.  Per-channel extremes are packed IEEE minimum/maximum (-0 below
// +0) over the lane's rows, reduced over the row groups in LDS; each channel
// gets its scale and zero once; codes use the exact quotient and go to LDS as
// bytes; key words are integer Horner over 4-digit chunks.
__device__ inline uint32_t u4_get16(const uint4& v, int i) {
  const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}
__device__ inline void u4_zero16(uint4& v, int i) {
  const uint32_t m = (i & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  if (i < 2) v.x &= m;
  else if (i < 4) v.y &= m;
  else if (i < 6) v.z &= m;
  else v.w &= m;
}
__device__ inline void top2_insert(uint32_t k, uint32_t& a1, uint32_t& a2) {
  a2 = max(a2, min(a1, k));
  a1 = max(a1, k);
}

struct KchanArgs {
  const uint16_t* k;
  int64_t sb, st, sh;
  int Hkv, tiles, kblocks, cap;
  uint32_t* kwords;
  uint32_t* kmeta;
  uint32_t* sparse;
};

template <int L, int SPV>
__global__ __launch_bounds__(256) void k_kchan_keys_fast(KchanArgs a) {
  using P = RowPack<L>;
  constexpr int KW = P::KW, CW = kD / 4 + 1;
  static_assert(SPV >= 0 && SPV <= 2, "at most two sparse entries per vector");
  __shared__ uint32_t codes[128][CW];
  __shared__ uint32_t red_mn[16][kD / 2], red_mx[16][kD / 2];
  __shared__ uint32_t cmeta[kD];
  __shared__ float crcp[kD];
  __shared__ int clamp_any;
  const int tid = threadIdx.x, l16 = tid & 15, rg = tid >> 4;
  const int blk = blockIdx.x, u = blockIdx.y;
  const int b = u / a.Hkv, h = u % a.Hkv;
  const int t0 = blk * 128;
  if (tid == 0) clamp_any = 0;
  const uint16_t* base = a.k + b * a.sb + h * a.sh + 8 * l16;
  uint4 x[8];
#pragma unroll
  for (int p = 0; p < 8; ++p)
    x[p] = *reinterpret_cast<const uint4*>(base + (int64_t)(t0 + 16 * p + rg) * a.st);
  // sparse entries: the SPV largest magnitudes of each row
  if (SPV > 0) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      uint32_t a1 = 0u, a2 = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t ch = 8 * l16 + i;
        top2_insert(((u4_get16(x[p], i) & 0x7FFFu) << 16) | (0xFFFFu - ch), a1, a2);
      }
      // merge with the partner's (disjoint) top two: pairs, quads, halves, rows
      auto merge = [&](uint32_t b1, uint32_t b2) {
        a2 = max(min(a1, b1), max(a2, b2));
        a1 = max(a1, b1);
      };
      merge(quad_perm<kQuadXor1>(a1), quad_perm<kQuadXor1>(a2));
      merge(quad_perm<kQuadXor2>(a1), quad_perm<kQuadXor2>(a2));
      merge(quad_perm<kRowHalfMirror>(a1), quad_perm<kRowHalfMirror>(a2));
      merge(quad_perm<kRowMirror>(a1), quad_perm<kRowMirror>(a2));
      const int c1 = 0xFFFF - (int)(a1 & 0xFFFFu), c2 = 0xFFFF - (int)(a2 & 0xFFFFu);
      const int t = t0 + 16 * p + rg;
      uint32_t* sp = a.sparse + ((size_t)u * a.cap + t) * SPV;
#pragma unroll
      for (int e = 0; e < SPV; ++e) {
        const int c = e == 0 ? c1 : c2;
        const int slot = SPV == 1 ? 0 : (c == min(c1, c2) ? 0 : 1);
        if ((c >> 3) == l16) {
          sp[slot] = ((uint32_t)c << 16) | u4_get16(x[p], c & 7);
          u4_zero16(x[p], c & 7);
        }
      }
    }
  }
  // per-channel extremes over the lane's rows, then over the row groups
  {
    uint32_t mn[4] = {x[0].x, x[0].y, x[0].z, x[0].w}, mx[4] = {x[0].x, x[0].y, x[0].z, x[0].w};
#pragma unroll
    for (int p = 1; p < 8; ++p) {
      const uint32_t w[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) { mn[k] = hmin(mn[k], w[k]); mx[k] = hmax(mx[k], w[k]); }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) { red_mn[rg][4 * l16 + k] = mn[k]; red_mx[rg][4 * l16 + k] = mx[k]; }
  }
  __syncthreads();
  if (tid < kD / 2) {
    uint32_t mn = red_mn[0][tid], mx = red_mx[0][tid];
#pragma unroll
    for (int r = 1; r < 16; ++r) { mn = hmin(mn, red_mn[r][tid]); mx = hmax(mx, red_mx[r][tid]); }
    bool sub = false;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = 2 * tid + e;
      const uint32_t cmn = e ? (mn >> 16) : (mn & 0xFFFFu), cmx = e ? (mx >> 16) : (mx & 0xFFFFu);
      GroupQ g = group_setup(cmn, cmx, L);
      if (g.s == 0.0f) g.r = 0.0f;
      const uint32_t meta = g.s_bits | (cmn << 16);
      a.kmeta[((size_t)u * a.kblocks + blk) * kD + ch] = meta;
      cmeta[ch] = meta;
      crcp[ch] = g.r;
      sub |= (g.s_bits & 0x7C00u) == 0u && g.s != 0.0f;
    }
    if (sub) atomicOr(&clamp_any, 1);
  }
  __syncthreads();
  {
    float one = 1.0f;
    asm volatile("" : "+v"(one));
    uint32_t m[8];
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { m[i] = cmeta[8 * l16 + i]; r[i] = crcp[8 * l16 + i]; }
    // the top-level clamp matters only where some scale is subnormal
    const float top = clamp_any != 0 ? (float)(L - 1) : INFINITY;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t w[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
      uint32_t c[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const h2v zs = hb(m[e]);                       // (s, z)
        const float q = fminf(quotient_of(hb(w[e / 2])[e & 1], zs[1], zs[0], r[e], one), top);
        c[e / 4] = __builtin_amdgcn_cvt_pk_u8_f32(q, e & 3, c[e / 4]);
      }
      codes[16 * p + rg][2 * l16] = c[0];
      codes[16 * p + rg][2 * l16 + 1] = c[1];
    }
  }
  __syncthreads();
  if (tid < 128) {
    const int s = t0 + tid;
    uint32_t row[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) row[j] = codes[tid][j];
    uint32_t* dst = a.kwords + (((size_t)u * a.tiles + s / kTile) * KW) * kTile + (s % kTile);
#pragma unroll
    for (int w = 0; w < KW; ++w) dst[w * kTile] = P::key_word(row, w);
  }
}

template <int L>
static bool launch_kchan_keys_L(const KchanArgs& a, int spv, dim3 grid, hipStream_t s) {
  switch (spv) {
    case 0: k_kchan_keys_fast<L, 0><<<grid, 256, 0, s>>>(a); return true;
    case 1: k_kchan_keys_fast<L, 1><<<grid, 256, 0, s>>>(a); return true;
    case 2: k_kchan_keys_fast<L, 2><<<grid, 256, 0, s>>>(a); return true;
  }
  return false;
}

static bool launch_kchan_keys_fast(const KchanArgs& a, int L, int spv, dim3 grid, hipStream_t s) {
  switch (L) {
    case 3: return launch_kchan_keys_L<3>(a, spv, grid, s);
    case 4: return launch_kchan_keys_L<4>(a, spv, grid, s);
    case 5: return launch_kchan_keys_L<5>(a, spv, grid, s);
    case 6: return launch_kchan_keys_L<6>(a, spv, grid, s);
    case 7: return launch_kchan_keys_L<7>(a, spv, grid, s);
    case 8: return launch_kchan_keys_L<8>(a, spv, grid, s);
  }
  return false;
}

// Copies the last nwin tokens of every unit into the fp16 window (zeros
// past them) and, in workgroup (0, 0), sets the per-sequence counters.
__global__ __launch_bounds__(256) void k_kchan_window(const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int64_t sb,
                                                      int64_t st, int64_t sh, int Hkv, int nq,
                                                      int nwin, int win_cap,
                                                      uint16_t* __restrict__ kwin,
                                                      uint16_t* __restrict__ vwin,
                                                      int32_t* __restrict__ counters, int B) {
  const int u = blockIdx.y;
  const int b = u / Hkv, h = u % Hkv;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int s = threadIdx.x; s < B; s += 256) {
      counters[s * 4 + 0] = nq + nwin;
      counters[s * 4 + 1] = nq;
      counters[s * 4 + 2] = nwin;
      counters[s * 4 + 3] = 0;
    }
  for (int e = blockIdx.x * 256 + threadIdx.x; e < win_cap * (kD / 8); e += gridDim.x * 256) {
    const int i = e / (kD / 8), c8 = (e % (kD / 8)) * 8;
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (i < nwin) {
      const int64_t off = b * sb + (int64_t)(nq + i) * st + h * sh + c8;
      kr = *reinterpret_cast<const uint4*>(k + off);
      vr = *reinterpret_cast<const uint4*>(v + off);
    }
    const size_t o = ((size_t)u * win_cap + i) * kD + c8;
    *reinterpret_cast<uint4*>(kwin + o) = kr;
    *reinterpret_cast<uint4*>(vwin + o) = vr;
  }
}

bool launch_quantize_kchan(const kvq_layout* L, uint8_t* cache, const void* k, const void* v,
                           int64_t sb, int64_t st, int64_t sh, int T, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const kvq_config& c = L->cfg;
  const int U = c.batch * c.kv_heads;
  const int nq = kchan_nq(L, T);
  const int nwin = T - nq;
  if (nwin > L->win_cap) return false;
  // the window kernel also resets the counters, so it runs before the value
  // quantizer, which may set a flag in them
  k_kchan_window<<<dim3(std::max(1, ceil_div(L->win_cap * (kD / 8), 256)), U), 256, 0, s>>>(
      (const uint16_t*)k, (const uint16_t*)v, sb, st, sh, c.kv_heads, nq, nwin, L->win_cap,
      (uint16_t*)(cache + L->k_win), (uint16_t*)(cache + L->v_win),
      (int32_t*)(cache + L->counters), c.batch);
  if (nq > 0) {
    KchanArgs ka;
    ka.k = (const uint16_t*)k;
    ka.sb = sb; ka.st = st; ka.sh = sh;
    ka.Hkv = c.kv_heads; ka.tiles = L->tiles[0]; ka.kblocks = L->kblocks; ka.cap = c.capacity;
    ka.kwords = (uint32_t*)(cache + L->k_words[0]);
    ka.kmeta = (uint32_t*)(cache + L->k_meta[0]);
    ka.sparse = (uint32_t*)(cache + L->sparse);
    const dim3 grid(nq / c.k_block, U);
    if (!launch_kchan_keys_fast(ka, c.k_levels, c.sparse_per_vec, grid, s))
      k_kchan_keys<<<grid, 256, 0, s>>>(
        (const uint16_t*)k, sb, st, sh, c.kv_heads, c.k_levels, L->nv[0], L->kw[0], L->tiles[0],
        L->kblocks, c.capacity, c.sparse_per_vec, (uint32_t*)(cache + L->k_words[0]),
        (uint32_t*)(cache + L->k_meta[0]), (uint32_t*)(cache + L->sparse));
  }
  QuantArgs a;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.sb = sb; a.st = st; a.sh = sh;
  a.inv = nullptr;
  a.inv_cap = 0;
  a.n = nq;
  a.L = c.v_levels; a.nv = L->vnv; a.kw = 0; a.tiles = L->tiles[0]; a.vrows = L->vrows[0];
  a.Hkv = c.kv_heads;
  a.kwords = nullptr;
  a.kmeta = nullptr;
  a.vwords = (uint32_t*)(cache + L->v_words[0]);
  a.vmeta = (uint32_t*)(cache + L->v_meta[0]);
  a.counters = (int32_t*)(cache + L->counters);
  if (!launch_pool(a, c.v_group, U, s)) return false;
  return hipGetLastError() == hipSuccess;
}

// --------------------------------------------------------------- append ----
// One workgroup per sequence.  Reads the running median, decides the tier,
// quantizes the new K and V rows of every KV head on that grid, writes them
// at the tier's next slot, inserts the score into the sorted array and bumps
// the counters.
struct AppendArgs {
  int32_t* counters;
  uint32_t* tokmap;
  float* sorted;
  uint32_t* kwords[2];
  uint32_t* kmeta[2];
  uint32_t* vwords[2];
  uint32_t* vmeta[2];
  const uint16_t* k_new;
  const uint16_t* v_new;
  const float* score_new;
  int L[2], nv[2], kw[2], tiles[2], vrows[2], cap[2];
  int capacity, Hkv, G;
  const uint8_t* korder = nullptr;   // [Hkv][128] stored channel orders, or null
  const uint8_t* vorder = nullptr;
  float clip = 1.0f;                 // group min/max scale factor (1: none)
  int skvq = 0;                      // orders or clipping in use
  int32_t* spos[2] = {nullptr, nullptr};   // pre-RoPE keys: token position of each slot
};

// One group of a new token's row with a stored channel order (ord: the
// group's G order bytes, or null for natural order) and a clipped range;
// codes in stored order to LDS, (scale, zero) returned.
template <int G>
__device__ inline uint32_t quant_group_skvq(const uint16_t* __restrict__ row, const uint8_t* ord, int g,
                                            float clip, int L, uint8_t* codes) {
  uint16_t x[G];
#pragma unroll
  for (int i = 0; i < G; ++i) x[i] = row[ord ? (int)(ord[i] & 0x7F) : g * G + i];
  int kmn = f16_order_key(x[0]), kmx = kmn;
#pragma unroll
  for (int i = 1; i < G; ++i) {
    const int kk = f16_order_key(x[i]);
    kmn = min(kmn, kk);
    kmx = max(kmx, kk);
  }
  uint32_t mn = f16_from_order_key(kmn), mx = f16_from_order_key(kmx);
  clip_range(mn, mx, clip);
  const GroupQ gq = group_setup(mn, mx, L);
#pragma unroll
  for (int i = 0; i < G; ++i) codes[i] = (uint8_t)quant_value(h2f(x[i]), gq);
  return gq.s_bits | (mn << 16);
}

constexpr int kAppendThreads = 1024;
constexpr int kAppendPerThread = 20;                  // sorted scores per thread per pass
constexpr int kAppendPass = kAppendThreads * kAppendPerThread;

// One workgroup per sequence.  The sorted scores are moved in passes of
// kAppendPass elements from the top down: a pass is read whole into registers
// before any of it is written, so a score greater than the new one can move up
// by one place in the same pass (a lower pass's writes end where this pass
// begins, after this pass has read it).  The scores at most equal to the new
// one stay; their count is the new score's position.
template <int G>
__global__ __launch_bounds__(kAppendThreads) void k_append(AppendArgs a) {
  constexpr int NG = kD / G;
  __shared__ int s_tier, s_slot, s_ok;
  __shared__ uint32_t s_le;
  __shared__ uint8_t codes[2][64][kD];     // [k/v][head][d], Hkv <= 64
  const int tid = threadIdx.x, b = blockIdx.x;
  int32_t* cnt = a.counters + b * 4;
  float* srt = a.sorted + (size_t)b * a.capacity;
  const float snew = a.score_new[b];
  const int len = cnt[0];
  float x[kAppendPerThread];
  auto load_pass = [&](int hi) {             // elements hi - 1 - tid - kAppendThreads k
#pragma unroll
    for (int k = 0; k < kAppendPerThread; ++k) {
      const int i = hi - 1 - tid - kAppendThreads * k;
      x[k] = i >= 0 ? srt[i] : 0.0f;
    }
  };
  if (tid == 0) {
    int tier = 0;                            // an empty sequence takes the hi grid
    if (len > 0) {
      const double m = ((double)srt[(len - 1) / 2] + (double)srt[len / 2]) * 0.5;
      tier = ((double)snew > m) ? 0 : 1;
    }
    const int slot = cnt[1 + tier];
    s_tier = tier;
    s_slot = slot;
    s_ok = (len < a.capacity && slot < a.cap[tier]) ? 1 : 0;
    s_le = 0;
  }
  load_pass(len);                            // the top pass, read while the tier is decided
  __syncthreads();
  if (!s_ok) {
    if (tid == 0) atomicOr(cnt + 3, kFlagPoolFull);
    return;
  }
  const int tier = s_tier, slot = s_slot;
  const int L = a.L[tier], nv = a.nv[tier], kw = a.kw[tier], tiles = a.tiles[tier],
            vrows = a.vrows[tier];
  uint32_t le = 0;
  for (int hi = len; hi > 0; hi -= kAppendPass) {
    if (hi != len) {
      load_pass(hi);
      __syncthreads();                       // the pass is read whole before it is written
    }
#pragma unroll
    for (int k = 0; k < kAppendPerThread; ++k) {
      const int i = hi - 1 - tid - kAppendThreads * k;
      if (i >= 0) {
        if (x[k] <= snew) ++le;
        else srt[i + 1] = x[k];
      }
    }
  }
  atomicAdd(&s_le, le);
  // quantize every (head, k/v, group)
  for (int task = tid; task < a.Hkv * 2 * NG; task += kAppendThreads) {
    const int h = task / (2 * NG), kv = (task / NG) % 2, g = task % NG;
    const uint16_t* row = (kv ? a.v_new : a.k_new) + ((size_t)b * a.Hkv + h) * kD;
    uint32_t meta;
    if (a.skvq) {
      const uint8_t* ord = kv ? a.vorder : a.korder;
      meta = quant_group_skvq<G>(row, ord ? ord + (size_t)h * kD + g * G : nullptr, g, a.clip, L,
                                 &codes[kv][h][g * G]);
    } else {
      meta = quant_group<G>(row + g * G, L, &codes[kv][h][g * G]);
    }
    const int u = b * a.Hkv + h;
    uint32_t* mp = kv ? a.vmeta[tier] : a.kmeta[tier];
    mp[(((size_t)u * tiles + slot / kTile) * NG + g) * kTile + (slot % kTile)] = meta;
    if (kv && (meta & 0x7FFFu) >= kBigScaleBits) atomicOr(cnt + 3, kFlagBigValueScale);
  }
  __syncthreads();
  const uint32_t pos = s_le;
  for (int task = tid; task < a.Hkv * kw; task += kAppendThreads) {
    const int h = task / kw, w = task % kw;
    const int u = b * a.Hkv + h;
    const int d0 = w * nv, d1 = min(kD, d0 + nv);
    uint32_t word = 0;
    for (int d = d1 - 1; d >= d0; --d) word = word * (uint32_t)L + codes[0][h][d];
    a.kwords[tier][(((size_t)u * tiles + slot / kTile) * kw + w) * kTile + (slot % kTile)] = word;
  }
  const int r = slot / nv, j = slot % nv;
  uint32_t pw = 1;
  for (int i = 0; i < j; ++i) pw *= (uint32_t)L;
  for (int task = tid; task < a.Hkv * kD; task += kAppendThreads) {
    const int h = task / kD, d = task % kD;
    const int u = b * a.Hkv + h;
    uint32_t* wp = &a.vwords[tier][((size_t)u * vrows + r) * kD + d];
    *wp = *wp + pw * (uint32_t)codes[1][h][d];
  }
  if (tid == 0) {                            // after every move (the barrier above)
    if (a.spos[tier]) a.spos[tier][(size_t)b * a.cap[tier] + slot] = len;
    srt[pos] = snew;
    a.tokmap[(size_t)b * a.capacity + len] = (uint32_t)slot | ((uint32_t)tier << 31);
    cnt[0] = len + 1;
    cnt[1 + tier] = slot + 1;
  }
}

bool launch_append(const kvq_layout* L, uint8_t* cache, const void* k_new, const void* v_new,
                   const float* score_new, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const kvq_config& c = L->cfg;
  if (c.kv_heads > 64) return false;
  AppendArgs a;
  a.counters = (int32_t*)(cache + L->counters);
  a.tokmap = (uint32_t*)(cache + L->tokmap);
  a.sorted = (float*)(cache + L->sorted);
  for (int p = 0; p < 2; ++p) {
    a.kwords[p] = (uint32_t*)(cache + L->k_words[p]);
    a.kmeta[p] = (uint32_t*)(cache + L->k_meta[p]);
    a.vwords[p] = (uint32_t*)(cache + L->v_words[p]);
    a.vmeta[p] = (uint32_t*)(cache + L->v_meta[p]);
    a.nv[p] = L->nv[p]; a.kw[p] = L->kw[p]; a.tiles[p] = L->tiles[p];
    a.vrows[p] = L->vrows[p]; a.cap[p] = L->cap[p];
    a.spos[p] = L->slot_pos[p] ? (int32_t*)(cache + L->slot_pos[p]) : nullptr;
  }
  a.L[0] = c.levels_hi;
  a.L[1] = c.levels_lo;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.score_new = score_new;
  a.capacity = c.capacity;
  a.Hkv = c.kv_heads;
  a.G = c.group;
  a.korder = c.reorder ? cache + L->chan_order : nullptr;
  a.vorder = c.reorder ? cache + L->chan_order + (size_t)c.kv_heads * kD : nullptr;
  a.clip = c.clip > 0.0f ? c.clip : 1.0f;
  a.skvq = (c.reorder || a.clip != 1.0f) ? 1 : 0;
  switch (c.group) {
    case 32: k_append<32><<<c.batch, kAppendThreads, 0, s>>>(a); break;
    case 64: k_append<64><<<c.batch, kAppendThreads, 0, s>>>(a); break;
    case 128: k_append<128><<<c.batch, kAppendThreads, 0, s>>>(a); break;
    default: return false;
  }
  return hipGetLastError() == hipSuccess;
}

// ------------------------------------------------------- channel orders ----
struct OrderBytes {
  uint32_t k[kD / 4], v[kD / 4];
};

__global__ __launch_bounds__(64) void k_write_order(uint32_t* dk, uint32_t* dv, OrderBytes o) {
  const int t = threadIdx.x;
  if (t < kD / 4) dk[t] = o.k[t];
  else if (t < kD / 2) dv[t - kD / 4] = o.v[t - kD / 4];
}

bool launch_write_order(uint8_t* dk, uint8_t* dv, const uint8_t* kbytes, const uint8_t* vbytes,
                        void* stream) {
  OrderBytes o;
  memcpy(o.k, kbytes, kD);
  memcpy(o.v, vbytes, kD);
  k_write_order<<<1, 64, 0, (hipStream_t)stream>>>((uint32_t*)dk, (uint32_t*)dv, o);
  return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
