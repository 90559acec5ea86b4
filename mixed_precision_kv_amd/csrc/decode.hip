// Decode attention over the packed cache, split over the context
// (SemKV, Abstract: attention reads every kept token of the compressed cache;
// KVQuant summary: small-batch decode is bound by memory bandwidth, so the
// packed words are read once and dequantized in registers).
//
// Grid: one workgroup per (context chunk, unit, pool).  Each computes, for the
// four query heads of its KV head, the chunk's running max m (log2 domain),
// the sum l of exp2(score - m) and the unnormalized sum of exp2(score - m) * v^,
// then a merge kernel combines every chunk of both pools (log-sum-exp).
//
// Scores use the group identity
//   q . k^ = sum_g ( s_g * sum_{d in g} q_d c_d  +  z_g * sum_{d in g} q_d )
// so keys are never dequantized value by value.
#include <string.h>

#include <atomic>

#include "common.h"
#include "internal.h"

namespace kvq {

constexpr int kDecThreads = 256;
constexpr int kPartStride = 4 + kD;        // floats per head: m, l, pad, pad, acc[128]
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const int32_t* counters;
  const uint16_t* q;
  float* part;
  int Hkv, nch_total, nch0;
  float scale_log2;
  // tiered pools / kchan quantized part
  const uint32_t* kwords[2];
  const uint32_t* kmeta[2];
  const uint32_t* vwords[2];
  const uint32_t* vmeta[2];
  int L[2], nv[2], kw[2], tiles[2], vrows[2], chunk[2];
  int group;
  // kchan extras
  const uint32_t* sparse;
  const uint16_t* kwin;
  const uint16_t* vwin;
  int vL, vnv, vgroup, spv, cap, kblocks, win_cap;
  int nwch;               // kchan: window chunks of kWinChunk tokens
};

// sum over the 16 lanes of a DPP row (every lane gets it)
__device__ inline float row_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x121, 0xF, 0xF, false));
  return v;
}

__device__ inline float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Softmax of the chunk's scores (sc[4][n], log2-scaled) in place -> p; returns
// per-head m, l in sm[4], sl[4].  Wave w handles head w.
__device__ inline void chunk_softmax(float (*sc)[640], int n, float* sm, float* sl) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float m = -INFINITY;
  for (int i = lane; i < n; i += 64) m = fmaxf(m, sc[w][i]);
  m = wave_max(m);
  float l = 0.f;
  for (int i = lane; i < n; i += 64) {
    float p = exp2f(sc[w][i] - m);
    sc[w][i] = p;
    l += p;
  }
  l = wave_sum(l);
  if (lane == 0) { sm[w] = m; sl[w] = l; }
}

__device__ inline void write_empty(float* part) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kGqa * kPartStride; i += kDecThreads) {
    const int j = i % kPartStride;
    part[i] = (j == 0) ? -INFINITY : 0.0f;
  }
}

// Value pass shared by every quantized layout: column words of nv slots,
// per-slot (scale, zero) in 16-slot tiles with groups of G along head_dim.
__device__ inline void value_pass(const uint32_t* __restrict__ vw, const uint32_t* __restrict__ vm,
                                  int u, int vrows, int tiles, int L, int nv, int G, int s_begin,
                                  int s_end, float (*p)[640], float* red, float* acc_out) {
  const int tid = threadIdx.x, d = tid & (kD - 1), half = tid >> 7;
  const int NG = kD / G, g = d / G;
  float acc[kGqa] = {0.f, 0.f, 0.f, 0.f};
  const int r_begin = s_begin / nv, r_end = ceil_div(s_end, nv);
  for (int r = r_begin + half; r < r_end; r += 2) {
    uint32_t word = vw[((size_t)u * vrows + r) * kD + d];
    for (int j = 0; j < nv; ++j) {
      const int s = r * nv + j;
      if (s >= s_end) break;
      const uint32_t c = word % (uint32_t)L;
      word /= (uint32_t)L;
      const uint32_t meta = vm[(((size_t)u * tiles + s / kTile) * NG + g) * kTile + (s % kTile)];
      const float v = __builtin_fmaf((float)c, h2f(meta & 0xFFFFu), h2f(meta >> 16));
      const int i = s - s_begin;
#pragma unroll
      for (int hh = 0; hh < kGqa; ++hh) acc[hh] = __builtin_fmaf(p[hh][i], v, acc[hh]);
    }
  }
  if (half == 1)
    for (int hh = 0; hh < kGqa; ++hh) red[hh * kD + d] = acc[hh];
  __syncthreads();
  if (half == 0)
    for (int hh = 0; hh < kGqa; ++hh) acc_out[hh * kD + d] = acc[hh] + red[hh * kD + d];
}

__device__ inline void finish_partial(float* part, const float* sm, const float* sl,
                                      const float* acc) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kGqa * kD; i += kDecThreads) {
    const int hh = i / kD, d = i % kD;
    part[hh * kPartStride + 4 + d] = acc[hh * kD + d];
  }
  if (tid < kGqa) {
    part[tid * kPartStride + 0] = sm[tid];
    part[tid * kPartStride + 1] = sl[tid];
  }
}

__device__ inline void load_q(const uint16_t* q, int b, int hk, int Hkv, float (*qf)[kD]) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kGqa * kD; i += kDecThreads) {
    const int hh = i / kD, d = i % kD;
    qf[hh][d] = h2f(q[((size_t)b * Hkv * kGqa + hk * kGqa + hh) * kD + d]);
  }
}

// Per-channel-key cache on the VALU, for the shapes the matrix-core kernel
// does not cover: blockIdx.z == 0 -> chunk blockIdx.x of the quantized tokens
// (per-channel keys + sparse), blockIdx.z == 1 -> chunk blockIdx.x of the
// fp16 window (kWinChunk tokens).
__global__ __launch_bounds__(kDecThreads) void k_decode_kchan(DecodeArgs a) {
  __shared__ float qf[kGqa][kD];
  __shared__ float qs[kGqa][kD];            // q * per-channel scale of the current key block
  __shared__ float qz[kGqa];
  __shared__ float sc[kGqa][640];
  __shared__ float red[kGqa * kD];
  __shared__ float accs[kGqa * kD];
  __shared__ float sm[kGqa], sl[kGqa];
  const int tid = threadIdx.x;
  const int c = blockIdx.x, u = blockIdx.y, z = blockIdx.z;
  const int b = u / a.Hkv, hk = u % a.Hkv;
  const int nchp = z ? a.nwch : a.nch0;
  if (c >= nchp) return;
  float* part = a.part + ((size_t)u * a.nch_total + (z ? a.nch0 : 0) + c) * kGqa * kPartStride;
  if (z == 1) {
    // window chunk c: tokens [kWinChunk c, kWinChunk (c + 1)) of the fp16 window.
    // Every row of the window's capacity is read before the valid count
    // arrives (rows past it are masked below), then the query
    const int w0 = c * kWinChunk, ncap = min(kWinChunk, a.win_cap - w0);
    const uint16_t* kwp = a.kwin + ((size_t)u * a.win_cap + w0) * kD;
    const uint16_t* vwp = a.vwin + ((size_t)u * a.win_cap + w0) * kD;
    // scores: sixteen lanes per token (one DPP row), eight channels each
    static_assert(kWinChunk * 16 == kDecThreads, "one 16-lane row per window token");
    const int i = tid >> 4, c8 = tid & 15;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
    if (i < ncap) kv = *reinterpret_cast<const uint4*>(kwp + (size_t)i * kD + 8 * c8);
    // values: thread (half, d) takes tokens half, half + 2, ...
    const int d = tid & (kD - 1), half = tid >> 7;
    uint16_t vr[kWinChunk / 2];
#pragma unroll
    for (int k = 0; k < kWinChunk / 2; ++k) {
      const int t = half + 2 * k;
      vr[k] = t < ncap ? vwp[(size_t)t * kD + d] : (uint16_t)0;
    }
    const int nwin_c = min(kWinChunk, a.counters[b * 4 + 2] - w0);
    if (nwin_c <= 0) { write_empty(part); return; }
    load_q(a.q, b, hk, a.Hkv, qf);
    __syncthreads();
    {
      const uint32_t wv[4] = {kv.x, kv.y, kv.z, kv.w};
      float sco[kGqa] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = h2f(e & 1 ? (wv[e / 2] >> 16) : (wv[e / 2] & 0xFFFFu));
#pragma unroll
        for (int hh = 0; hh < kGqa; ++hh) sco[hh] = __builtin_fmaf(qf[hh][8 * c8 + e], x, sco[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < kGqa; ++hh) {
        const float t = row_sum16(sco[hh]);
        if (c8 == 0) sc[hh][i] = i < nwin_c ? t * a.scale_log2 : -INFINITY;
      }
    }
    __syncthreads();
    chunk_softmax(sc, nwin_c, sm, sl);
    __syncthreads();
    float acc[kGqa] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kWinChunk / 2; ++k) {
      const int t = half + 2 * k;
      if (t < nwin_c) {
        const float vv = h2f(vr[k]);
        for (int hh = 0; hh < kGqa; ++hh) acc[hh] = __builtin_fmaf(sc[hh][t], vv, acc[hh]);
      }
    }
    if (half == 1)
      for (int hh = 0; hh < kGqa; ++hh) red[hh * kD + d] = acc[hh];
    __syncthreads();
    if (half == 0)
      for (int hh = 0; hh < kGqa; ++hh) accs[hh * kD + d] = acc[hh] + red[hh * kD + d];
    __syncthreads();
    finish_partial(part, sm, sl, accs);
    return;
  }
  const int nq = a.counters[b * 4 + 1];
  load_q(a.q, b, hk, a.Hkv, qf);
  __syncthreads();
  const int CH = a.chunk[0];
  const int s_begin = c * CH, s_end = min(nq, s_begin + CH);
  if (s_begin >= s_end) { write_empty(part); return; }
  const int L = a.L[0], nv = a.nv[0], kw = a.kw[0], tiles = a.tiles[0];
  for (int blk0 = s_begin; blk0 < s_end; blk0 += 128) {
    const int kb = blk0 / 128;
    for (int i = tid; i < kGqa * kD; i += kDecThreads) {
      const int hh = i / kD, d = i % kD;
      const uint32_t meta = a.kmeta[0][((size_t)u * a.kblocks + kb) * kD + d];
      qs[hh][d] = qf[hh][d] * h2f(meta & 0xFFFFu);
      red[i] = qf[hh][d] * h2f(meta >> 16);
    }
    __syncthreads();
    if (tid < kGqa) {
      float sz = 0.f;
      for (int d = 0; d < kD; ++d) sz += red[tid * kD + d];
      qz[tid] = sz;
    }
    __syncthreads();
    if (tid < 128) {
      const int s = blk0 + tid;
      float sco[kGqa] = {0.f, 0.f, 0.f, 0.f};
      const uint32_t* kp = a.kwords[0] + ((size_t)u * tiles + s / kTile) * kw * kTile + (s % kTile);
      for (int w = 0; w < kw; ++w) {
        uint32_t word = kp[w * kTile];
        for (int j = 0; j < nv; ++j) {
          const int d = w * nv + j;
          if (d >= kD) break;
          const float cf = (float)(word % (uint32_t)L);
          word /= (uint32_t)L;
          for (int hh = 0; hh < kGqa; ++hh) sco[hh] = __builtin_fmaf(qs[hh][d], cf, sco[hh]);
        }
      }
      for (int e = 0; e < a.spv; ++e) {
        const uint32_t ent = a.sparse[((size_t)u * a.cap + s) * a.spv + e];
        const int ch = ent >> 16;
        const float val = h2f(ent & 0xFFFFu);
        for (int hh = 0; hh < kGqa; ++hh) sco[hh] = __builtin_fmaf(qf[hh][ch], val, sco[hh]);
      }
      for (int hh = 0; hh < kGqa; ++hh) sc[hh][s - s_begin] = (sco[hh] + qz[hh]) * a.scale_log2;
    }
    __syncthreads();
  }
  chunk_softmax(sc, s_end - s_begin, sm, sl);
  __syncthreads();
  value_pass(a.vwords[0], a.vmeta[0], u, a.vrows[0], tiles, a.vL, a.vnv, a.vgroup, s_begin, s_end,
             sc, red, accs);
  __syncthreads();
  finish_partial(part, sm, sl, accs);
}

// Merge of the chunk partials: a partial per (unit, chunk, head) is the
// chunk's running max m_c, its sum l_c, two pad words and the 128 sums
// (132 floats, 16-byte aligned).
constexpr int kMergeBatch = 8;                // chunks per thread per round trip

// Chunks c0, c0 + step, ... (< nch) of one head, partials at pu with cs
// floats between chunks, into (M, lsum, o): a batch's loads are issued
// before any is used; the running max grows batch by batch, rescaling what
// has been summed.  Lane q owns channels 4q .. 4q + 3.
__device__ inline void merge_accumulate(const float* __restrict__ pu, size_t cs, int c0, int step, int nch,
                                        int q, float& M, float& lsum, float4& o) {
  for (int cb = c0; cb < nch; cb += step * kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    float4 av[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int c = cb + k * step;
      const bool ok = c < nch;
      const float* pc = pu + (size_t)(ok ? c : 0) * cs;
      mv[k] = ok ? pc[0] : -INFINITY;
      lv[k] = pc[1];
      av[k] = *reinterpret_cast<const float4*>(pc + 4 + 4 * q);
    }
    float mb = M;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) mb = fmaxf(mb, mv[k]);
    const float f = (M == -INFINITY) ? 0.f : exp2f(M - mb);   // rescale of what is summed so far
    lsum *= f;
    o.x *= f; o.y *= f; o.z *= f; o.w *= f;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float w = (mv[k] == -INFINITY) ? 0.f : exp2f(mv[k] - mb);
      lsum = __builtin_fmaf(lv[k], w, lsum);
      o.x = __builtin_fmaf(av[k].x, w, o.x);
      o.y = __builtin_fmaf(av[k].y, w, o.y);
      o.z = __builtin_fmaf(av[k].z, w, o.z);
      o.w = __builtin_fmaf(av[k].w, w, o.w);
    }
    M = mb;
  }
}

// Lane q's four channels of one head's output r / l as fp16; position p of
// the sums is channel vorder_h[p] of the output (stored value order).
__device__ inline void merge_write(uint16_t* __restrict__ po, const uint8_t* __restrict__ vorder_h, int q,
                                   float4 r, float l) {
  const uint32_t ch = vorder_h ? *reinterpret_cast<const uint32_t*>(vorder_h + 4 * q) & 0x7F7F7F7Fu
                               : 0x03020100u + 0x04040404u * (uint32_t)q;
  po[ch & 0xFF] = f2h_rne(r.x / l);
  po[(ch >> 8) & 0xFF] = f2h_rne(r.y / l);
  po[(ch >> 16) & 0xFF] = f2h_rne(r.z / l);
  po[ch >> 24] = f2h_rne(r.w / l);
}

// Log-sum-exp merge of every chunk partial of one (unit, head) -> fp16 output,
// in one pass.  Thread (slice sl, quad q) owns chunks c = sl, sl + S, ... and
// channels 4q..4q+3; the slices are combined through LDS against the largest
// max.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void k_merge(const float* __restrict__ part,
                                                   uint16_t* __restrict__ out, int nch_total,
                                                   int Hkv, float2* __restrict__ stats,
                                                   const uint8_t* __restrict__ vorder) {
  constexpr int S = THREADS / 32;             // slices
  __shared__ float smax[S];
  __shared__ float4 racc[S][32];
  __shared__ float rl[S];
  const int u = blockIdx.x, hh = blockIdx.y, t = threadIdx.x;
  const int b = u / Hkv, hk = u % Hkv;
  const float* pu = part + (size_t)u * nch_total * kGqa * kPartStride + hh * kPartStride;
  const size_t cs = (size_t)kGqa * kPartStride;
  const int q = t & 31, sl = t >> 5;
  float M = -INFINITY, lsum = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  merge_accumulate(pu, cs, sl, S, nch_total, q, M, lsum, o);
  if (q == 0) smax[sl] = M;
  __syncthreads();
  float Mg = smax[0];
#pragma unroll
  for (int k = 1; k < S; ++k) Mg = fmaxf(Mg, smax[k]);
  const float f = (M == -INFINITY) ? 0.f : exp2f(M - Mg);
  racc[sl][q] = make_float4(o.x * f, o.y * f, o.z * f, o.w * f);
  if (q == 0) rl[sl] = lsum * f;
  __syncthreads();
  if (t < 32) {
    float4 r = racc[0][t];
    float l = rl[0];
#pragma unroll
    for (int k = 1; k < S; ++k) {
      const float4 x = racc[k][t];
      r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
      l += rl[k];
    }
    uint16_t* po = out + ((size_t)b * Hkv * kGqa + hk * kGqa + hh) * kD;
    if (stats && t == 0) stats[u * kGqa + hh] = make_float2(Mg, l);   // (max, sum) of the head
    merge_write(po, vorder ? vorder + (size_t)hk * kD : nullptr, t, r, l);
  }
}

// Many chunks over few units: the same merge with each head's 128 channels
// split over four workgroups of 256 threads (32 slices x 8 lanes of four
// channels), so that four times as many CUs share the partial reads.
__global__ __launch_bounds__(256) void k_merge_q(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                 int nch_total, int Hkv, float2* __restrict__ stats,
                                                 const uint8_t* __restrict__ vorder) {
  constexpr int S = 32;                      // slices
  __shared__ float smax[S];
  __shared__ float4 racc[S][8];
  __shared__ float rl[S];
  const int u = blockIdx.x, hh = blockIdx.y, cq = blockIdx.z, t = threadIdx.x;
  const int b = u / Hkv, hk = u % Hkv;
  const float* pu = part + (size_t)u * nch_total * kGqa * kPartStride + hh * kPartStride;
  const size_t cs = (size_t)kGqa * kPartStride;
  const int ql = t & 7, sl = t >> 3, q = 8 * cq + ql;   // q: quad of channels 4q .. 4q + 3
  float M = -INFINITY, lsum = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  merge_accumulate(pu, cs, sl, S, nch_total, q, M, lsum, o);
  if (ql == 0) smax[sl] = M;
  __syncthreads();
  float Mg = smax[0];
#pragma unroll
  for (int k = 1; k < S; ++k) Mg = fmaxf(Mg, smax[k]);
  const float f = (M == -INFINITY) ? 0.f : exp2f(M - Mg);
  racc[sl][ql] = make_float4(o.x * f, o.y * f, o.z * f, o.w * f);
  if (ql == 0) rl[sl] = lsum * f;
  __syncthreads();
  if (t < 8) {
    float4 r = racc[0][t];
    float l = rl[0];
#pragma unroll
    for (int k = 1; k < S; ++k) {
      const float4 x = racc[k][t];
      r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
      l += rl[k];
    }
    uint16_t* po = out + ((size_t)b * Hkv * kGqa + hk * kGqa + hh) * kD;
    if (stats && cq == 0 && t == 0) stats[u * kGqa + hh] = make_float2(Mg, l);   // (max, sum) of the head
    merge_write(po, vorder ? vorder + (size_t)hk * kD : nullptr, q, r, l);
  }
}

// Few chunks per unit: one workgroup of 128 threads per unit; lane (head
// t / 32, quad t % 32) merges every chunk of its head by itself (one slice,
// no LDS combine), so a unit costs two waves instead of four workgroups.
__global__ __launch_bounds__(128) void k_merge_unit(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                    int nch_total, int Hkv, float2* __restrict__ stats,
                                                    const uint8_t* __restrict__ vorder) {
  const int u = blockIdx.x, t = threadIdx.x, hh = t >> 5, q = t & 31;
  const int b = u / Hkv, hk = u % Hkv;
  const float* pu = part + (size_t)u * nch_total * kGqa * kPartStride + hh * kPartStride;
  float M = -INFINITY, lsum = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  merge_accumulate(pu, (size_t)kGqa * kPartStride, 0, 1, nch_total, q, M, lsum, o);
  if (stats && q == 0) stats[u * kGqa + hh] = make_float2(M, lsum);
  merge_write(out + ((size_t)b * Hkv * kGqa + hk * kGqa + hh) * kD, vorder ? vorder + (size_t)hk * kD : nullptr,
              q, o, lsum);
}

// One slice per head for a batch of chunks or two, 8 slices for more, 32 for
// many (long contexts over few units)
static void launch_merge(const float* part, uint16_t* out, int U, int nch, int Hkv, hipStream_t s,
                         float2* stats = nullptr, const uint8_t* vorder = nullptr) {
  if (nch <= 2 * kMergeBatch)
    k_merge_unit<<<U, 128, 0, s>>>(part, out, nch, Hkv, stats, vorder);
  else if (nch <= 8 * kMergeBatch)
    k_merge<256><<<dim3(U, kGqa), 256, 0, s>>>(part, out, nch, Hkv, stats, vorder);
  else
    k_merge_q<<<dim3(U, kGqa, 4), 256, 0, s>>>(part, out, nch, Hkv, stats, vorder);
}

// Attention mass of every cached token of sequence b: the softmax weight it
// receives summed over the sequence's query heads, from the pools' raw
// (log2-domain) scores and each head's (max, sum) after the merge; the token
// map gives each token's pool and slot.  Tokens past the sequence's length
// get 0.
__global__ __launch_bounds__(256) void k_token_mass(const int32_t* __restrict__ counters,
                                                   const uint32_t* __restrict__ tokmap,
                                                   const float* __restrict__ raw0,
                                                   const float* __restrict__ raw1,
                                                   const float2* __restrict__ stats,
                                                   float* __restrict__ mass, int cap, int cap0,
                                                   int cap1, int Hkv, int max_len) {
  const int b = blockIdx.y, t = blockIdx.x * 256 + threadIdx.x;
  if (t >= max_len) return;
  float sum = 0.f;
  if (t < counters[b * 4 + 0]) {
    const uint32_t mp = tokmap[(size_t)b * cap + t];
    const bool lo = (mp >> 31) != 0u;
    const uint32_t slot = mp & 0x7FFFFFFFu;
    const float* raw = lo ? raw1 : raw0;
    const int capp = lo ? cap1 : cap0;
    for (int hk = 0; hk < Hkv; ++hk) {
      const int u = b * Hkv + hk;
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        const float2 st = stats[u * kGqa + h];
        sum += __builtin_amdgcn_exp2f(raw[((size_t)u * kGqa + h) * capp + slot] - st.x) / st.y;
      }
    }
  }
  mass[(size_t)b * max_len + t] = sum;
}

// Partial bytes a decode of sequences of at most max_len tokens writes with
// the chunk split launch_decode chooses (decode_ws_bytes bounds every split).
// The tiered decode's split: both pools in one launch of npair chunks per
// unit (npair > 0), else nchp[p] chunks of chunk[p] slots per pool.
struct TieredSplit {
  int npair, chunk[2], nchp[2];
  int used() const { return npair > 0 ? npair : nchp[0] + nchp[1]; }
};
static TieredSplit tiered_split(const kvq_layout* L, int max_len) {
  const kvq_config& c = L->cfg;
  const int U = c.batch * c.kv_heads;
  const int lv[2] = {c.levels_hi, c.levels_lo};
  int slots[2];
  for (int p = 0; p < 2; ++p) slots[p] = L->cap[p] < max_len ? L->cap[p] : max_len;
  TieredSplit t;
  memset(&t, 0, sizeof(t));
  // pre-RoPE keys keep one launch per pool (the pair kernel has no rotation)
  if (!L->slot_pos[0] && !L->slot_pos[1])
    t.npair = decode_pair_chunks(lv[0], lv[1], c.group, U, slots[0], slots[1]);
  if (t.npair == 0)
    for (int p = 0; p < 2; ++p) {
      t.chunk[p] = decode_pool_chunk(lv[p], c.group, U, slots[p], L->slot_pos[p] != 0);
      t.nchp[p] = ceil_div(slots[p], t.chunk[p]);
    }
  return t;
}

size_t decode_ws_used(const kvq_layout* L, int max_len) {
  const kvq_config& c = L->cfg;
  const size_t U = (size_t)c.batch * c.kv_heads;
  int nch0, nch1;
  int nch = decode_chunks(L, max_len, &nch0, &nch1);
  if (c.mode == KVQ_MODE_TIERED) nch = tiered_split(L, max_len).used();
  return U * nch * kGqa * kPartStride * 4;
}

size_t decode_ws_bytes(const kvq_layout* L, int max_len, bool mass) {
  int a, b;
  const int n = decode_chunks(L, max_len, &a, &b);
  const size_t U = (size_t)L->cfg.batch * L->cfg.kv_heads;
  size_t bytes = U * n * kGqa * kPartStride * 4;
  if (mass) bytes += U * kGqa * ((size_t)L->cap[0] + L->cap[1]) * 4 + U * kGqa * 8;
  return bytes;
}

kvq_status launch_decode(const kvq_layout* L, const uint8_t* cache, const void* q, float scale,
                         int max_len, void* out, uint8_t* ws, void* stream, float* mass) {
  hipStream_t s = (hipStream_t)stream;
  const kvq_config& c = L->cfg;
  const int U = c.batch * c.kv_heads;
  int nch0, nch1;
  const int nch = decode_chunks(L, max_len, &nch0, &nch1);
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.counters = (const int32_t*)(cache + L->counters);
  a.q = (const uint16_t*)q;
  a.part = (float*)ws;
  a.Hkv = c.kv_heads;
  a.nch_total = nch;
  a.nch0 = nch0;
  a.scale_log2 = scale * kLog2e;
  if (c.mode == KVQ_MODE_TIERED) {
    const int lv[2] = {c.levels_hi, c.levels_lo};
    const TieredSplit sp = tiered_split(L, max_len);
    const int nch_used = sp.used();
    if (nch_used > nch) return KVQ_ERR_WORKSPACE;   // the workspace holds the finest split
    // with the token mass: raw scores of both pools, then per-head (max, sum)
    float* raw[2];
    raw[0] = (float*)(ws + (size_t)U * nch * kGqa * kPartStride * 4);
    raw[1] = raw[0] + (size_t)U * kGqa * L->cap[0];
    float2* stats = (float2*)(raw[1] + (size_t)U * kGqa * L->cap[1]);
    const uint8_t* korder = c.reorder ? cache + L->chan_order : nullptr;
    const uint8_t* vorder = c.reorder ? korder + (size_t)c.kv_heads * kD : nullptr;
    PoolArgs pargs[2];
    for (int p = 0; p < 2; ++p) {
      PoolArgs& pa = pargs[p];
      pa.counters = a.counters;
      pa.q = a.q;
      pa.part = a.part;
      pa.kwords = (const uint32_t*)(cache + L->k_words[p]);
      pa.kmeta = (const uint32_t*)(cache + L->k_meta[p]);
      pa.vwords = (const uint32_t*)(cache + L->v_words[p]);
      pa.vmeta = (const uint32_t*)(cache + L->v_meta[p]);
      pa.pool = p;
      pa.Hkv = c.kv_heads;
      pa.tiles = L->tiles[p];
      pa.vrows = L->vrows[p];
      pa.nch_total = nch_used;
      pa.part_off = sp.npair > 0 ? 0 : p ? sp.nchp[0] : 0;
      pa.chunk = sp.chunk[p];
      pa.c = a.scale_log2;
      pa.raw = mass ? raw[p] : nullptr;
      pa.cap_p = L->cap[p];
      pa.korder = korder;
      pa.spos = L->slot_pos[p] ? (const int32_t*)(cache + L->slot_pos[p]) : nullptr;
      pa.rope_theta = c.rope_theta;
      if (sp.npair == 0 && sp.nchp[p] > 0 && !launch_decode_pool(lv[p], pa, c.group, sp.nchp[p], U, stream))
        return KVQ_ERR_LAUNCH;
    }
    if (sp.npair > 0 && !launch_decode_pair(lv[0], lv[1], c.group, pargs[0], pargs[1], sp.npair, U, stream))
      return KVQ_ERR_LAUNCH;
    launch_merge((const float*)ws, (uint16_t*)out, U, nch_used, c.kv_heads, s, mass ? stats : nullptr,
                 vorder);
    if (mass)
      k_token_mass<<<dim3(ceil_div(max_len, 256), c.batch), 256, 0, s>>>(
          a.counters, (const uint32_t*)(cache + L->tokmap), raw[0], raw[1], stats, mass, c.capacity,
          L->cap[0], L->cap[1], c.kv_heads, max_len);
    return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
  } else {
    a.kwords[0] = (const uint32_t*)(cache + L->k_words[0]);
    a.kmeta[0] = (const uint32_t*)(cache + L->k_meta[0]);
    a.vwords[0] = (const uint32_t*)(cache + L->v_words[0]);
    a.vmeta[0] = (const uint32_t*)(cache + L->v_meta[0]);
    a.L[0] = c.k_levels; a.nv[0] = L->nv[0]; a.kw[0] = L->kw[0]; a.tiles[0] = L->tiles[0];
    a.vrows[0] = L->vrows[0];
    a.chunk[0] = decode_chunk_kchan(L);
    if (a.chunk[0] > 640) return KVQ_ERR_UNSUPPORTED;
    a.vL = c.v_levels; a.vnv = L->vnv; a.vgroup = c.v_group; a.spv = c.sparse_per_vec;
    a.cap = c.capacity; a.kblocks = L->kblocks; a.win_cap = L->win_cap;
    a.sparse = (const uint32_t*)(cache + L->sparse);
    a.nwch = nch1;
    a.kwin = (const uint16_t*)(cache + L->k_win);
    a.vwin = (const uint16_t*)(cache + L->v_win);
    if (L->win_cap > 640) return KVQ_ERR_UNSUPPORTED;
    if (!launch_decode_kchan_mfma(L, cache, q, a.scale_log2, a.part, nch0, nch1, nch, stream)) {
      const int gx = nch0 > nch1 ? nch0 : nch1;
      k_decode_kchan<<<dim3(gx, U, 2), kDecThreads, 0, s>>>(a);
    }
  }
  launch_merge((const float*)ws, (uint16_t*)out, U, nch, c.kv_heads, s);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

// ---- allocation-free decode ----
// The partials live in a fixed device array instead of a caller workspace.
// Host code never passes the array's name to a kernel: it is a host-side
// stand-in there.  The device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and is kept per device (each
// GPU holds its own copy of the array).  Every call on one GPU shares the
// array; the decode writes every partial it reads, so nothing needs clearing,
// and calls that overlap on one GPU race on it.
constexpr int kMaxScratchDevices = 64;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];
static std::atomic<uintptr_t> g_scratch_addr[kMaxScratchDevices];

static uint8_t* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    p = (uintptr_t)ptr;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  return (uint8_t*)p;
}

kvq_status launch_decode_noalloc(const kvq_layout* L, const uint8_t* cache, const void* q, float scale,
                                 int max_len, void* out, void* stream) {
  const size_t U = (size_t)L->cfg.batch * L->cfg.kv_heads;
  // every split needs at least one partial per unit and pool (checked before any HIP call)
  if (U * 2 * kGqa * kPartStride * 4 > kNoAllocScratchBytes) return KVQ_ERR_WORKSPACE;
  if (decode_ws_used(L, max_len) > kNoAllocScratchBytes) return KVQ_ERR_WORKSPACE;
  uint8_t* ws = scratch_ptr();
  if (!ws) return KVQ_ERR_LAUNCH;
  return launch_decode(L, cache, q, scale, max_len, out, ws, stream);
}

}  // namespace kvq
