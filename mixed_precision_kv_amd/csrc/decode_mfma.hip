// Decode attention over one tier pool on the matrix cores (gfx950
// v_mfma_f32_16x16x32_f16).  SemKV, Abstract: attention reads every kept
// token; KVQuant summary: small-batch decode is memory-bound, so packed words
// are read once and expanded in registers.
//
// One workgroup per (chunk of slots, sequence x KV head).  Per 16-slot key
// tile: lane (n = slot, j) owns row words j, j+4, j+8, ... of slot n; their
// base-L digits, as fp16, are the B operand directly.  The A operand is the
// query of the four heads spread over 16 rows (sub-group of 32 channels x
// head), zero outside its sub-group, so the result row (g, h) of column n is
// the partial dot sum_{d in g} q_h[d] c_d of slot n.  Lane (n, g) holds rows
// (g, 0..3) and the (scale, zero) of group g of slot n, so it forms
//     s_g * P + z_g * sum_{d in g} q_h[d]
// and a reduce-scatter across the four lanes of slot n (two permlane swaps)
// leaves lane (n, h) with the score of head h.
// Values are stored in column words (n_L consecutive slots of one channel),
// so the slot axis is the lane's contraction axis: B[k = slot][col = channel]
// comes straight out of the words; A[(g, h)][slot] = p_h * s_g(slot) is an
// fp16 product of the weight and the scale; the zero-point term sum p_h z_g
// is a dot product on the VALU.  Online softmax (base 2) per macro tile;
// partials (m, l, acc) go to the workspace for the log-sum-exp merge.
#include <atomic>

#include "common.h"
#include "internal.h"
#include "tiling.h"
#include "unpack.h"
#include "mfma_util.h"

namespace kvq {

// Two waves per workgroup, one per load stream (the vector-memory counter is
// in-order, so each stream is issued in the order it is consumed):
//   wave 0 (keys)   macro tile i: scores, running max, weights p = 2^(s - m)
//                   as fp16 into an LDS double buffer (in the value
//                   operand's order), rescale factor alpha;
//   wave 1 (values) macro tile i-1: A = p * s from that buffer, column-word
//                   digits, matrix ops into the accumulators.
// One barrier per macro tile hands buffer (i & 1) from wave 0 to wave 1.
// ROPE (pre-RoPE keys, KVQuant summary "techniques"): the key wave turns
// every dequantized key by its token position before the dot product.  Per
// key tile the lane's expanded digits go to LDS in channel order; lane (n, j)
// then takes channels 32 j .. 32 j + 31 of slot n (16 adjacent pairs),
// dequantizes them in fp32, turns pair i by position * theta_i (the angle in
// revolutions, reduced mod 1 in 32-bit fixed point from a 64-bit fraction
// theta_i / 2 pi, then the hardware sine and cosine), and hands
// the rotated key to the matrix cores as fp16 high and low parts against A
// rows 4h .. 4h + 3 = query head h, so lane (n, j) receives head j's score.
// Softmax and value sums a workgroup carries from one pool's pass to the
// next (lane (n, h) of the key wave; the value wave's accumulator rows).
// The value sums are in units of `mul`, the digit multiplier of the pass
// that formed them: the output row is ((acc - asum) mul + zacc) / 2^6 (times
// 2^6 again for a sequence flagged for large value scales).
struct PassCarry {
  float m_run, l_run;
  f4 acc[8];
  f4 asum;
  float zacc;
  float mul;
};

__device__ __forceinline__ void carry_init(PassCarry& cr, float mul) {
  cr.m_run = -INFINITY;
  cr.l_run = 0.f;
#pragma unroll
  for (int v = 0; v < 8; ++v) cr.acc[v] = (f4){0.f, 0.f, 0.f, 0.f};
  cr.asum = (f4){0.f, 0.f, 0.f, 0.f};
  cr.zacc = 0.f;
  cr.mul = mul;
}

// One pool's slots [s_begin, s_end) of unit blockIdx.y (s_begin < s_end),
// added to the carried softmax and sums.  Every thread of the workgroup
// calls it; each wave takes its own branch, with the same number of
// workgroup barriers in both.
template <int L, int G, bool ROPE>
__device__ __forceinline__ void pool_pass(const PoolArgs& a, int s_begin, int s_end, PassCarry& cr) {
  using T = Tiling<L>;
  constexpr int NV = T::NV, KW = T::KW, KWL = T::KWL, R = T::R, RUN = T::RUN, MT = T::MT,
                KT = T::KT;
  using DK = Unpack<L, KWL>;                 // key words of one lane
  using DV = Unpack<L, R>;                   // value words of one lane and channel tile
  constexpr int KM = DK::NH8, VM = DV::NH8;
  constexpr bool AFF = DK::kAffine;
  constexpr float MUL = (float)DK::kMul;
  constexpr int NG = kD / G;                 // (scale, zero) groups per row
  constexpr int SUB = G / 32;                // 32-channel sub-groups per group
  constexpr int VK = VM * 8;                 // padded slot run per lane group
  constexpr int META = KT * NG * 16;         // (scale, zero) words per macro tile
  constexpr int META_PER_LANE = (META + 63) / 64;

  __shared__ float qf[kGqa][kD];
  __shared__ __attribute__((aligned(16))) _Float16 pw_lds[2][kGqa][4 * VK];  // 2^6 p, operand order (wave 0 -> 1)
  __shared__ float al_lds[2][kGqa];          // rescale factor per head
  __shared__ __attribute__((aligned(16))) _Float16 vs_lds[NG][4 * VK];  // value scale, operand order
  __shared__ __attribute__((aligned(16))) _Float16 vz_lds[NG][4 * VK];  // value zero, same order
  __shared__ int ppos_lds[MT];               // slot -> position in that order
  __shared__ int mpos_lds[64 * META_PER_LANE];
  __shared__ uint2 ctab[DK::kTableEntries];   // chunk -> four fp16 digits
  __shared__ uint2 rev_lds[ROPE ? kD / 2 : 1];    // theta_i / 2 pi as a 64-bit binary fraction (hi, lo)
  __shared__ __attribute__((aligned(16))) _Float16 kc_lds[ROPE ? 16 : 1][ROPE ? kD + 8 : 1];  // a key tile, channel order

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;    // B/C-operand view: slot/channel n, group j
  const int u = blockIdx.y;
  const int b = u / a.Hkv, hk = u % a.Hkv;
  const int nmt = (s_end - s_begin + MT - 1) / MT;

  // ---- shared set-up
  // q in stored channel order: position d holds channel korder[d] (7-bit)
  for (int i = threadIdx.x; i < kGqa * kD; i += 128) {
    const int d = i % kD, src = a.korder ? (int)(a.korder[(size_t)hk * kD + d] & 0x7F) : d;
    qf[i / kD][d] = h2f(a.q[((size_t)b * a.Hkv * kGqa + hk * kGqa + i / kD) * kD + src]);
  }
  for (int sl = threadIdx.x; sl < MT; sl += 128) {
    const int jj = sl / RUN, rem = sl % RUN;
    ppos_lds[sl] = jj * VK + DV::pos_of(rem / NV, rem % NV);
  }
  for (int e = threadIdx.x; e < 64 * META_PER_LANE; e += 128) {
    const int ee = min(e, META - 1);
    const int sl = (ee / (NG * 16)) * 16 + (ee % 16);
    const int jj = sl / RUN, rem = sl % RUN;
    mpos_lds[e] = jj * VK + DV::pos_of(rem / NV, rem % NV);
  }
  DK::fill(ctab, threadIdx.x, 128);
  if (ROPE && threadIdx.x < kD / 2) {
    // revolutions per position, f = theta_i / 2 pi < 1/(2 pi), split exactly
    // into its first 64 fraction bits (f * 2^32 and its remainder are exact
    // in fp64)
    const double f = exp2(-(double)(2 * threadIdx.x) / kD * log2((double)a.rope_theta)) *
                     0.15915494309189533577;   // / (2 pi)
    const double f32 = f * 4294967296.0, fh = floor(f32);
    rev_lds[threadIdx.x] = make_uint2((uint32_t)fh, (uint32_t)floor((f32 - fh) * 4294967296.0));
  }
  // operand positions that hold no slot keep weight and scale 0
  for (int i = threadIdx.x; i < 4 * VK; i += 128) {
    for (int h = 0; h < 4; ++h) { pw_lds[0][h][i] = (_Float16)0.0f; pw_lds[1][h][i] = (_Float16)0.0f; }
    for (int g = 0; g < NG; ++g) { vs_lds[g][i] = (_Float16)0.0f; vz_lds[g][i] = (_Float16)0.0f; }
  }
  __syncthreads();

  if (wave == 0) {
    // ================= keys: scores, softmax, weights =================
    // The key wave's long dependent chain (table reads, matrix ops, lane
    // reduction per tile) sets the pace of the pair; it gets the higher
    // issue priority so the value waves sharing its SIMD fill the gaps.
    __builtin_amdgcn_s_setprio(3);
    const BufRes rK = make_res(a.kwords + (size_t)u * a.tiles * KW * 16, a.tiles * KW * 16 * 4);
    const BufRes rKM = make_res(a.kmeta + (size_t)u * a.tiles * NG * 16, a.tiles * NG * 16 * 4);
    uint32_t kwoff[KWL];
#pragma unroll
    for (int wi = 0; wi < KWL; ++wi) {
      const int w = j + 4 * wi;
      kwoff[wi] = w < KW ? (uint32_t)(w * 16 + n) * 4u : kOutOfRange;
    }
    const uint32_t kmoff = (uint32_t)((j / SUB) * 16 + n) * 4u;
    const BufRes rSP = make_res(ROPE ? a.spos + (size_t)b * a.cap_p : a.counters, ROPE ? a.cap_p * 4 : 4);
    struct KBuf {
      uint32_t kw[KT][KWL];
      uint32_t km[KT];
      uint32_t pos[ROPE ? KT : 1];             // token positions of the tile's slots
    };
    auto load_k = [&](KBuf& kb, int s0) {
      const uint32_t tile0 = s0 / 16;
#pragma unroll
      for (int t = 0; t < KT; ++t) {
#pragma unroll
        for (int wi = 0; wi < KWL; ++wi) kb.kw[t][wi] = bload(rK, kwoff[wi] + (tile0 + t) * (KW * 16 * 4));
        kb.km[t] = bload(rKM, kmoff + (tile0 + t) * (NG * 16 * 4));
        if (ROPE) kb.pos[t] = bload(rSP, ((tile0 + t) * 16 + n) * 4u);
      }
    };
    KBuf nxt;
    load_k(nxt, s_begin);
    float qc[4];                             // lane (n, g): c * sum_{d in g} q_h[d]
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float sum = 0.f;
#pragma unroll
      for (int d = 0; d < 32; ++d) sum += qf[h][32 * j + d];
      qc[h] = sum * a.c;
    }
    h8 aq[KM];
    {
      const int r = n, g = r >> 2, h = r & 3;   // A-operand view: row r, k-range of group j
      const int nw = (KW - j + 3) / 4;          // words this lane group owns
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = 8 * m + i;
          const int wi = DK::word_of(t);
          const int d = (j + 4 * wi) * NV + DK::digit_of(t);
          const bool ok = wi >= 0 && wi < nw && d < kD && (d >> 5) == g;
          const float qv = qf[h][min(max(d, 0), kD - 1)];
          aq[m][i] = (_Float16)(ok ? qv : 0.0f);   // q is fp16: exact
        }
    }
    h8 aqr[ROPE ? 4 : 1];                    // rotated keys: A[r][k] = q_{r/4}[32 (k/8) + 8 m + k%8]
    if (ROPE) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) aqr[m][e] = (_Float16)qf[n >> 2][32 * j + 8 * m + e];
    }
    int spos[KT];                            // operand position of slot 16 t + n
#pragma unroll
    for (int t = 0; t < KT; ++t) spos[t] = ppos_lds[16 * t + n];
    // score of head j for slot n with the key turned by its position: the
    // expanded operand values v (digits, or 1 + d/MUL on power-of-two grids)
    // give the key sg v + zz
    auto rope_score = [&](const h8 (&bk)[KM], float sg, float zz, uint32_t pos) -> float {
      wave_lds_fence();                      // the previous tile's gather is done
#pragma unroll
      for (int m = 0; m < KM; ++m)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tt = 8 * m + i, wi = DK::word_of(tt);
          if (wi >= 0) {
            const int w = j + 4 * wi, d = w * NV + DK::digit_of(tt);
            if (w < KW && d < kD) kc_lds[n][d] = bk[m][i];
          }
        }
      wave_lds_fence();
      f4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const h8 cv = *reinterpret_cast<const h8*>(&kc_lds[n][32 * j + 8 * m]);
        h8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x = __builtin_fmaf(sg, (float)cv[e], zz);
          const float y = __builtin_fmaf(sg, (float)cv[e + 1], zz);
          // pos * f mod 1 in 32-bit fixed point: the low word of pos * hi
          // plus the carry of pos * lo (error below 2^-32 revolutions)
          const uint2 fr = rev_lds[16 * j + 4 * m + e / 2];
          const uint32_t t = pos * fr.x + __umulhi(pos, fr.y);
          const float rv = (float)t * 0x1p-32f;   // revolutions in [0, 1]
          const float cs = __builtin_amdgcn_cosf(rv), sn = __builtin_amdgcn_sinf(rv);
          const float xr = x * cs - y * sn, yr = x * sn + y * cs;
          hi[e] = (_Float16)xr;
          hi[e + 1] = (_Float16)yr;
          lo[e] = (_Float16)(xr - (float)hi[e]);
          lo[e + 1] = (_Float16)(yr - (float)hi[e + 1]);
        }
        pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqr[m], hi, pr, 0, 0, 0);
        pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(aqr[m], lo, pr, 0, 0, 0);
      }
      return pr[0];
    };
    float m_run = cr.m_run, l_run = cr.l_run;
    for (int it = 0; it <= nmt; ++it) {
      if (it < nmt) {
        const int s0 = s_begin + it * MT;
        const KBuf cur = nxt;
        if (it + 1 < nmt) load_k(nxt, s0 + MT);
        float scs[KT];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          h8 bk[KM];
          DK::run(cur.kw[t], ctab, bk);
          const uint32_t meta = cur.km[t];
          const float sg = h2f(meta & 0xFFFFu) * MUL;
          const float zz = AFF ? h2f(meta >> 16) - sg : h2f(meta >> 16);
          float sc;
          if constexpr (ROPE) {
            sc = rope_score(bk, sg, zz, cur.pos[t]) * a.c;
          } else {
            f4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < KM; ++m) pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[m], bk[m], pr, 0, 0, 0);
            const float ssc = sg * a.c;
            f4 x;
#pragma unroll
            for (int h = 0; h < 4; ++h) x[h] = __builtin_fmaf(ssc, pr[h], zz * qc[h]);
            sc = reduce_scatter4(x);
          }
          scs[t] = (s0 + 16 * t + n < s_end) ? sc : -INFINITY;
          mx = fmaxf(mx, scs[t]);
        }
        // raw scores after the tile loop: a branch inside it would cut the
        // six tiles into separate blocks that the scheduler cannot overlap
        if (a.raw) {
#pragma unroll
          for (int t = 0; t < KT; ++t)
            if (s0 + 16 * t + n < s_end)     // lane (n, j): head j of slot n
              a.raw[((size_t)u * kGqa + j) * a.cap_p + s0 + 16 * t + n] = scs[t];
        }
        // online softmax (lane (n, h): head h).  Weights go to the value wave
        // as fp16 2^6 p, rounded half up: add half an fp16 spacing to the fp32
        // bits, then the truncating conversion (unbiased, unlike truncation
        // alone, whose bias the cancellation between the value and zero-point
        // sums would amplify).  The 2^6 keeps small weights out of the fp16
        // subnormal range.
        mx = row_max16(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        _Float16* pb = &pw_lds[it & 1][j][0];
        float ls = 0.f;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const float p = __builtin_amdgcn_exp2f(scs[t] - m_use);
          ls += p;
          const float x = __uint_as_float(__float_as_uint(p * kAScale) + 0x1000u);
          pb[spos[t]] = __builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz(x, x))[0];
        }
        l_run = __builtin_fmaf(l_run, alpha, ls);
        m_run = m_new;
        if (n == 0) al_lds[it & 1][j] = alpha;
      }
      __syncthreads();
    }
    cr.m_run = m_run;
    cr.l_run = l_run;
  } else {
    // ================= values: A = p * s, matrix ops =================
    const BufRes rVM = make_res(a.vmeta + (size_t)u * a.tiles * NG * 16, a.tiles * NG * 16 * 4);
    const BufRes rV = make_res(a.vwords + (size_t)u * a.vrows * kD, a.vrows * kD * 4);
    int mpos[META_PER_LANE];
#pragma unroll
    for (int k = 0; k < META_PER_LANE; ++k) mpos[k] = mpos_lds[lane + 64 * k];
    struct VBuf {
      uint32_t vm[META_PER_LANE];
      uint32_t vw[8][R];
    };
    auto load_v = [&](VBuf& vb, int s0) {
      const uint32_t tile0 = s0 / 16;
#pragma unroll
      for (int k = 0; k < META_PER_LANE; ++k) {
        const int e = lane + 64 * k;
        const uint32_t off = (META % 64 == 0 || e < META) ? (tile0 * NG * 16 + e) * 4u : kOutOfRange;
        vb.vm[k] = bload(rVM, off);
      }
      const uint32_t row0 = s0 / NV + j * R;
#pragma unroll
      for (int v = 0; v < 8; ++v)
#pragma unroll
        for (int r2 = 0; r2 < R; ++r2) vb.vw[v][r2] = bload(rV, ((row0 + r2) * kD + 16 * v + n) * 4u);
    };
    VBuf nxt;
    load_v(nxt, s_begin);
    // value scales of 1024 and above (flagged per sequence by quantize and
    // append) enter the fp16 product divided by 2^6, so that 2^6 p * s stays
    // finite for every finite fp16 scale
    const bool vbig = (a.counters[b * 4 + 3] & kFlagBigValueScale) != 0;
    // A-operand view: lane (r, j) holds row r = (sub-group sg, head h) over
    // the operand positions of lane group j
    const int h = n & 3, g = (n >> 2) / SUB;
    float zacc = cr.zacc;                    // 2^6 sum p z (row r)
    f4 acc[8];
    f4 asum = cr.asum;                       // power-of-two grids: sum of A per row
    // sums carried from a pass on another grid: into this grid's units
    // (both multipliers are powers of two, so the rescale is exact)
    const float cfac = cr.mul / MUL;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      acc[v] = cr.acc[v];
      if (cfac != 1.0f)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[v][e] = (acc[v][e] - asum[e]) * cfac;
    }
    if (cfac != 1.0f) asum = (f4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it <= nmt; ++it) {
      if (it >= 1) {
        const int i = it - 1;
        const int s0 = s_begin + i * MT;
        const VBuf cur = nxt;
        if (i + 1 < nmt) load_v(nxt, s0 + MT);
        const float al0 = al_lds[i & 1][0], al1 = al_lds[i & 1][1];
        const float al2 = al_lds[i & 1][2], al3 = al_lds[i & 1][3];
        if (!(al0 == 1.f && al1 == 1.f && al2 == 1.f && al3 == 1.f)) {
          // acc rows are (sg, h) with h = register index
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            acc[v][0] *= al0; acc[v][1] *= al1; acc[v][2] *= al2; acc[v][3] *= al3;
          }
          if (AFF) { asum[0] *= al0; asum[1] *= al1; asum[2] *= al2; asum[3] *= al3; }
          const float alh = h == 0 ? al0 : h == 1 ? al1 : h == 2 ? al2 : al3;
          zacc *= alh;
        }
        // value (scale, zero) in operand order, as fp16.  Operand digits are
        // 1 + d/MUL on power-of-two grids; MUL and the affine offset (removed
        // through asum) are applied in fp32 at the end.  Only this wave uses
        // vs/vz; its LDS accesses execute in order.
#pragma unroll
        for (int k = 0; k < META_PER_LANE; ++k) {
          const int e = lane + 64 * k;
          if (META % 64 == 0 || e < META) {
            const int gg = (e / 16) % NG;
            const uint32_t mw = cur.vm[k];
            vs_lds[gg][mpos[k]] = value_scale_operand(mw, vbig);
            vz_lds[gg][mpos[k]] = __builtin_bit_cast(_Float16, (uint16_t)(mw >> 16));
          }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the stores above have landed
        __builtin_amdgcn_wave_barrier();
        h8 av[VM];
#pragma unroll
        for (int m = 0; m < VM; ++m) {
          const int pos = j * VK + 8 * m;
          const h8 p16 = *reinterpret_cast<const h8*>(&pw_lds[i & 1][h][pos]);
          const h8 sv = *reinterpret_cast<const h8*>(&vs_lds[g][pos]);
          const h8 zv = *reinterpret_cast<const h8*>(&vz_lds[g][pos]);
          av[m] = p16 * sv;                  // fp16 products, rounded to nearest
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            zacc = __builtin_amdgcn_fdot2((h2v){p16[e], p16[e + 1]}, (h2v){zv[e], zv[e + 1]}, zacc, false);
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          h8 bv[VM];
          DV::run(cur.vw[v], ctab, bv);
#pragma unroll
          for (int m = 0; m < VM; ++m) acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[m], bv[m], acc[v], 0, 0, 0);
        }
        if (AFF) {
          const h8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
          for (int m = 0; m < VM; ++m) asum = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[m], ones, asum, 0, 0, 0);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) cr.acc[v] = acc[v];
    cr.asum = asum;
    cr.zacc = zacc;
    cr.mul = MUL;
  }
}

// A chunk's partial (m, l, acc) per head from the carried state.
__device__ __forceinline__ void write_partial(const PoolArgs& a, float* part, const PassCarry& cr) {
  __shared__ float zred[16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  if (wave == 0) {
    const float l_tot = row_sum16(cr.l_run);
    if (n == 0) {
      part[j * kPartF + 0] = cr.m_run;
      part[j * kPartF + 1] = l_tot;
    }
  } else {
    const int b = (int)blockIdx.y / a.Hkv;
    const bool vbig = (a.counters[b * 4 + 3] & kFlagBigValueScale) != 0;
    // zacc: lanes (r, j) -> sum over j per row r = 4 sg + h
    float zs = cr.zacc;
    zs += __shfl_xor(zs, 16);
    zs += __shfl_xor(zs, 32);
    if (lane < 16) zred[lane] = zs;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // acc rows (sg = j, h) hold channels of sub-group j
    const float vfac = cr.mul * (vbig ? kBigValueShift : 1.0f);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      if ((v >> 1) != j) continue;           // channels 16v..16v+15 belong to sub-group v/2
      const int d = 16 * v + n;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float t = (cr.acc[v][hh] - cr.asum[hh]) * vfac + zred[4 * j + hh];
        part[hh * kPartF + 4 + d] = t * (1.0f / kAScale);
      }
    }
  }
}

__device__ __forceinline__ void write_empty_partial(float* part) {
  for (int i = threadIdx.x; i < kGqa * kPartF; i += 128) part[i] = (i % kPartF == 0) ? -INFINITY : 0.f;
}

// Slots [begin, end) of chunk c of gridDim.x over one pool: the unit's filled
// slots split evenly over the launch's chunks, in whole macro tiles (the grid
// is sized for the pool's capacity, which can exceed the filled slots by a
// whole chunk's share).
template <int L>
__device__ __forceinline__ int2 chunk_span(const PoolArgs& a, int c) {
  constexpr int MT = Tiling<L>::MT;
  const int b = (int)blockIdx.y / a.Hkv;
  const int n_valid = a.counters[b * 4 + 1 + a.pool];
  const int span = ((n_valid + MT - 1) / MT + (int)gridDim.x - 1) / (int)gridDim.x * MT;
  const int s_begin = c * span;
  return make_int2(s_begin, min(n_valid, s_begin + span));
}

template <int L, int G, bool ROPE>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void k_decode_pool(PoolArgs a) {
  const int c = blockIdx.x, u = blockIdx.y;
  float* part = a.part + ((size_t)u * a.nch_total + a.part_off + c) * kGqa * kPartF;
  const int2 sp = chunk_span<L>(a, c);
  if (sp.x >= sp.y) {
    write_empty_partial(part);
    return;
  }
  PassCarry cr;
  carry_init(cr, (float)Unpack<L, Tiling<L>::KWL>::kMul);
  pool_pass<L, G, ROPE>(a, sp.x, sp.y, cr);
  write_partial(a, part, cr);
}

// Both tier pools of a unit in one launch: chunk c of the launch takes chunk
// c of each pool's even split, the high pool first, and carries its softmax
// and value sums into the low pool's pass, so the workgroup writes one
// partial for both pools and the merge reads one partial per chunk.  Each
// pass keeps its own LDS arrays and does its own set-up.
template <int L0, int L1, int G>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void k_decode_pair(PoolArgs a0, PoolArgs a1) {
  const int c = blockIdx.x, u = blockIdx.y;
  float* part = a0.part + ((size_t)u * a0.nch_total + c) * kGqa * kPartF;
  const int2 s0 = chunk_span<L0>(a0, c), s1 = chunk_span<L1>(a1, c);
  if (s0.x >= s0.y && s1.x >= s1.y) {
    write_empty_partial(part);
    return;
  }
  PassCarry cr;
  carry_init(cr, (float)Unpack<L0, Tiling<L0>::KWL>::kMul);
  if (s0.x < s0.y) pool_pass<L0, G, false>(a0, s0.x, s0.y, cr);
  if (s1.x < s1.y) pool_pass<L1, G, false>(a1, s1.x, s1.y, cr);
  write_partial(a0, part, cr);
}

// At three waves per SIMD (six workgroups per CU: the 6-level pool with
// 32-channel groups) the two waves of a workgroup land on two SIMDs so that
// half the SIMDs hold two key waves and a value wave and half one key wave
// and two value waves; the key waves of the latter run about 15 % slower and
// set the launch's end.  This instance therefore takes extra dynamic LDS
// (unused) up to 38 KB per workgroup, so that four fit a CU: one key and
// one value wave on every SIMD.  With pre-RoPE keys the rotation needs the
// third wave, so that instance keeps it.
constexpr int kFourPerCuLds = 38 * 1024;
template <int L, int G>
static size_t pad_lds() {
  if (!(L == 6 && G == 32)) return 0;
  static std::atomic<int> pad{-1};
  int v = pad.load(std::memory_order_relaxed);
  if (v < 0) {
    hipFuncAttributes at;
    v = (hipFuncGetAttributes(&at, reinterpret_cast<const void*>(&k_decode_pool<L, G, false>)) == hipSuccess &&
         (int)at.sharedSizeBytes < kFourPerCuLds)
            ? kFourPerCuLds - (int)at.sharedSizeBytes
            : 0;
    pad.store(v, std::memory_order_relaxed);
  }
  return (size_t)v;
}

template <int L, int G>
static void launch_one(const PoolArgs& a, int nch, int U, hipStream_t s) {
  if (a.spos)
    k_decode_pool<L, G, true><<<dim3(nch, U), 128, 0, s>>>(a);
  else
    k_decode_pool<L, G, false><<<dim3(nch, U), 128, pad_lds<L, G>(), s>>>(a);
}

template <int L, int G>
static int occupancy_one(bool rope) {
  int blocks = 0;
  const hipError_t e =
      rope ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pool<L, G, true>, 128, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pool<L, G, false>, 128, pad_lds<L, G>());
  return e == hipSuccess ? blocks : 0;
}

template <int L>
static bool launch_L(const PoolArgs& a, int G, int nch, int U, hipStream_t s) {
  switch (G) {
    case 32: launch_one<L, 32>(a, nch, U, s); return true;
    case 64: launch_one<L, 64>(a, nch, U, s); return true;
    case 128: launch_one<L, 128>(a, nch, U, s); return true;
  }
  return false;
}

template <int L>
static int occupancy_L(int G, bool rope) {
  switch (G) {
    case 32: return occupancy_one<L, 32>(rope);
    case 64: return occupancy_one<L, 64>(rope);
    case 128: return occupancy_one<L, 128>(rope);
  }
  return 0;
}

static int occupancy(int L, int G, bool rope) {
  switch (L) {
    case 3: return occupancy_L<3>(G, rope);
    case 4: return occupancy_L<4>(G, rope);
    case 5: return occupancy_L<5>(G, rope);
    case 6: return occupancy_L<6>(G, rope);
    case 7: return occupancy_L<7>(G, rope);
    case 8: return occupancy_L<8>(G, rope);
  }
  return 0;
}

// Per-device caches of the CU count and of the pool kernels' occupancy
// (value + 1; 0: not read yet).  Threads that race on a first read compute
// the same value, so relaxed atomics suffice.
constexpr int kMaxDevices = 64;
static std::atomic<int> g_cus[kMaxDevices];
static std::atomic<int> g_occ[kMaxDevices][9][3][2];

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int cus = cached ? g_cus[dev].load(std::memory_order_relaxed) - 1 : -1;
  if (cus < 0) {
    int n = 0;
    cus = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
    if (cached) g_cus[dev].store(cus + 1, std::memory_order_relaxed);
  }
  return cus;
}

int chunk_for_one_round(int L, int U, int slots_per_unit, int blocks_per_cu) {
  const int mt = macro_tile_slots(L);
  const long waves = (long)device_cu_count() * blocks_per_cu;
  if (waves <= 0 || slots_per_unit <= 0) return 8 * mt;
  // macro tiles per workgroup so that U * chunks ~ the resident workgroups
  const long tiles_per_unit = (slots_per_unit + mt - 1) / mt;
  long m = (tiles_per_unit * U + waves - 1) / waves;
  if (m < 1) m = 1;
  if (m > tiles_per_unit) m = tiles_per_unit;
  return (int)(m * mt);
}

int decode_pool_chunk(int L, int G, int U, int slots_per_unit, bool rope) {
  const int gi = G == 32 ? 0 : G == 64 ? 1 : 2;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < kMaxDevices && L >= 0 && L <= 8;
  int occ = cached ? g_occ[dev][L][gi][rope].load(std::memory_order_relaxed) - 1 : -1;
  if (occ < 0) {
    occ = occupancy(L, G, rope);
    if (cached) g_occ[dev][L][gi][rope].store(occ + 1, std::memory_order_relaxed);
  }
  return chunk_for_one_round(L, U, slots_per_unit, occ);
}

// ---- both tier pools in one launch (k_decode_pair) for the level pairs the
// workloads use; other pairs launch one kernel per pool
static int pair_index(int L0, int L1, int G) {
  if (L0 == 6 && L1 == 5 && G == 32) return 0;
  if (L0 == 8 && L1 == 6 && G == 64) return 1;
  return -1;
}
static std::atomic<int> g_occ_pair[kMaxDevices][2];

int decode_pair_chunks(int L0, int L1, int G, int U, int slots0, int slots1) {
  const int k = pair_index(L0, L1, G);
  if (k < 0 || U <= 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int occ = cached ? g_occ_pair[dev][k].load(std::memory_order_relaxed) - 1 : -1;
  if (occ < 0) {
    int blocks = 0;
    const hipError_t e = k == 0 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pair<6, 5, 32>, 128, 0)
                                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pair<8, 6, 64>, 128, 0);
    occ = e == hipSuccess ? blocks : 0;
    if (cached) g_occ_pair[dev][k].store(occ + 1, std::memory_order_relaxed);
  }
  const long resident = (long)device_cu_count() * occ;
  if (resident <= 0) return 0;
  // one round of resident workgroups, at most one chunk per macro tile of the
  // larger pool
  const long t0 = (slots0 + macro_tile_slots(L0) - 1) / macro_tile_slots(L0);
  const long t1 = (slots1 + macro_tile_slots(L1) - 1) / macro_tile_slots(L1);
  long nch = resident / U;
  if (nch > (t0 > t1 ? t0 : t1)) nch = t0 > t1 ? t0 : t1;
  return nch < 1 ? 1 : (int)nch;
}

bool launch_decode_pair(int L0, int L1, int G, const PoolArgs& a0, const PoolArgs& a1, int nch, int U,
                        void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (pair_index(L0, L1, G)) {
    case 0: k_decode_pair<6, 5, 32><<<dim3(nch, U), 128, 0, s>>>(a0, a1); return true;
    case 1: k_decode_pair<8, 6, 64><<<dim3(nch, U), 128, 0, s>>>(a0, a1); return true;
  }
  return false;
}

bool launch_decode_pool(int L, const PoolArgs& a, int G, int nch, int U, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  switch (L) {
    case 3: return launch_L<3>(a, G, nch, U, s);
    case 4: return launch_L<4>(a, G, nch, U, s);
    case 5: return launch_L<5>(a, G, nch, U, s);
    case 6: return launch_L<6>(a, G, nch, U, s);
    case 7: return launch_L<7>(a, G, nch, U, s);
    case 8: return launch_L<8>(a, G, nch, U, s);
  }
  return false;
}

// ===================== per-channel keys on the matrix cores =====================
// Quantized part of the per-channel-key cache (KVQuant summary, "techniques":
// per-channel keys in 128-token blocks, per-vector dense-and-sparse outliers;
// SKVQ, Abstract: 2-bit keys) for 4-level keys, 3-level values and value
// groups of 32.  A workgroup (four waves) owns a 640-token chunk: five key
// blocks, forty key tiles, four value units of 160 slots.
//   keys:   each wave scores ten 16-token tiles.  The per-channel scale sits
//           in the A operand: row 2h holds fp16(4 q_h[d] s_d) and row 2h + 1
//           the fp16 remainder of 4 q_h[d] s_d (exact in fp32), so hi + lo
//           carries the product to about 2^-22 and both land in one lane of
//           the result; the digits as fp16 are 1 + c/4,
//           and sum_d q_h[d] (z_d - 4 s_d) per block is added in fp32, as are
//           the sparse entries q_h[ch] * value.
//   softmax over the chunk's 640 scores (wave h: head h), weights 2^6 p as
//           fp16 rounded half up, in the value operand's order.
//   values: wave w runs value unit w through the same column-word matrix
//           path as the tiered pools; the four units are summed in LDS.
struct KchanDecArgs {
  const int32_t* counters;
  const uint16_t* q;
  float* part;
  const uint32_t* kwords;       // [u][tile][8][16]
  const uint32_t* kmeta;        // [u][key block][128]
  const uint32_t* sparse;       // [u][cap][spv]
  const uint32_t* vwords;       // [u][row][128]
  const uint32_t* vmeta;        // [u][tile][NG][16]
  const uint16_t* kwin;         // fp16 window [u][win_cap][128]
  const uint16_t* vwin;
  int Hkv, tiles, kblocks, vrows, cap, spv, nch_total;
  int nch0, win_cap;            // quantized chunks per unit; window capacity
  float c;                      // softmax scale * log2(e)
};

constexpr int kKcCH = 640, kKcKB = 128, kKcNB = kKcCH / kKcKB, kKcTW = kKcCH / 16 / 4;

// Chunk c of the fp16 window (tokens kWinChunk c ..), as extra workgroups of
// the same launch.  Scores: sixteen lanes per token (one DPP row), eight
// channels each; values: thread (half, d) takes tokens half, half + 2, ...
// Rows up to the window's capacity are read before the valid count arrives
// (rows past it are masked), then the query.  lds: 4 x 16 scores, then
// 4 x 128 partial sums.
__device__ inline void kchan_window_chunk(const KchanDecArgs& a, int c, int u, int b, int hk,
                                          float (*qf)[kD], float* lds, float* hm, float* hl) {
  static_assert(kWinChunk * 16 == 256, "one 16-lane row per window token");
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float (*wsc)[kWinChunk] = reinterpret_cast<float (*)[kWinChunk]>(lds);
  float (*wred)[kD] = reinterpret_cast<float (*)[kD]>(lds + kGqa * kWinChunk);
  float* part = a.part + ((size_t)u * a.nch_total + a.nch0 + c) * kGqa * kPartF;
  const int w0 = c * kWinChunk, ncap = min(kWinChunk, a.win_cap - w0);
  const uint16_t* kwp = a.kwin + ((size_t)u * a.win_cap + w0) * kD;
  const uint16_t* vwp = a.vwin + ((size_t)u * a.win_cap + w0) * kD;
  const int i = tid >> 4, c8 = tid & 15;
  uint4 kv = make_uint4(0u, 0u, 0u, 0u);
  if (i < ncap) kv = *reinterpret_cast<const uint4*>(kwp + (size_t)i * kD + 8 * c8);
  const int d = tid & (kD - 1), half = tid >> 7;
  uint16_t vr[kWinChunk / 2];
#pragma unroll
  for (int k = 0; k < kWinChunk / 2; ++k) {
    const int t = half + 2 * k;
    vr[k] = t < ncap ? vwp[(size_t)t * kD + d] : (uint16_t)0;
  }
  const int nwin_c = min(kWinChunk, a.counters[b * 4 + 2] - w0);
  if (nwin_c <= 0) {
    for (int e = tid; e < kGqa * kPartF; e += 256) part[e] = (e % kPartF == 0) ? -INFINITY : 0.f;
    return;
  }
  for (int e = tid; e < kGqa * kD; e += 256)
    qf[e / kD][e % kD] = h2f(a.q[((size_t)b * a.Hkv * kGqa + hk * kGqa) * kD + e]);
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
      if (c8 == 0) wsc[hh][i] = i < nwin_c ? t * a.c : -INFINITY;
    }
  }
  __syncthreads();
  {
    // softmax of head w over the chunk: lanes 0..15 of wave w
    const float x = wsc[w][lane & 15];
    const float mx = row_max16(x);
    const float p = __builtin_amdgcn_exp2f(x - mx);
    const float l = row_sum16(p);
    if (lane < kWinChunk) wsc[w][lane] = p;
    if (lane == 0) { hm[w] = mx; hl[w] = l; }
  }
  __syncthreads();
  float acc[kGqa] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kWinChunk / 2; ++k) {
    const int t = half + 2 * k;
    if (t < nwin_c) {
      const float vv = h2f(vr[k]);
#pragma unroll
      for (int hh = 0; hh < kGqa; ++hh) acc[hh] = __builtin_fmaf(wsc[hh][t], vv, acc[hh]);
    }
  }
  if (half == 1)
#pragma unroll
    for (int hh = 0; hh < kGqa; ++hh) wred[hh][d] = acc[hh];
  __syncthreads();
  if (half == 0)
#pragma unroll
    for (int hh = 0; hh < kGqa; ++hh) part[hh * kPartF + 4 + d] = acc[hh] + wred[hh][d];
  if (tid < kGqa) {
    part[tid * kPartF + 0] = hm[tid];
    part[tid * kPartF + 1] = hl[tid];
  }
}

template <int VL, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_decode_kchan_mfma(KchanDecArgs a) {
  using DKc = Digits<4, 2>;                  // key words j and j + 4 of a lane
  constexpr int NVV = cpw(VL), R = 2, VU = 4 * R * NVV;
  using DV = Unpack<VL, R>;
  constexpr int VM = DV::NH8, VK = VM * 8, NG = kD / G;
  static_assert(VU * 4 == kKcCH, "one value unit per wave");
  static_assert(VK == R * DV::PW || !DV::kTable, "value operand without padding");
  static_assert(G == 32, "value groups of 32 channels");
  __shared__ float qf[kGqa][kD];
  __shared__ float aoff[kKcNB][kGqa];
  __shared__ uint2 ctab[DV::kTableEntries];
  __shared__ float zr[4][16];
  __shared__ float hm[kGqa], hl[kGqa];
  // Two overlays (each region's users are separated by a barrier):
  //   A: key-operand tables and staged key scales (set-up, keys), then the
  //      value weights, scales and zeros (softmax, values);
  //   B: the chunk's scores (keys, softmax), then the per-wave outputs.
  typedef _Float16 Atab[kKcNB][4][4][8][8];               // [blk][m][j][row][i]
  typedef _Float16 VOp[4 * 4 * VK];
  constexpr int kAKey = sizeof(Atab) + kKcNB * kKcKB * 4;
  constexpr int kAVal = (kGqa + 2 * NG) * (int)sizeof(VOp);
  constexpr int kB = (kGqa * kKcCH > 4 * kGqa * kD ? kGqa * kKcCH : 4 * kGqa * kD) * 4;
  __shared__ __attribute__((aligned(16))) uint8_t ovA[kAKey > kAVal ? kAKey : kAVal];
  __shared__ __attribute__((aligned(16))) uint8_t ovB[kB];
  Atab& atab = *reinterpret_cast<Atab*>(ovA);
  uint32_t* kms = reinterpret_cast<uint32_t*>(ovA + sizeof(Atab));
  VOp* pw = reinterpret_cast<VOp*>(ovA);                      // [kGqa]
  VOp* vsl = pw + kGqa;                                       // [NG]
  VOp* vzl = vsl + NG;                                        // [NG]
  float (*sc)[kKcCH] = reinterpret_cast<float (*)[kKcCH]>(ovB);
  float (*red)[kGqa][kD] = reinterpret_cast<float (*)[kGqa][kD]>(ovB);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const int u = blockIdx.y;
  const int b = u / a.Hkv, hk = u % a.Hkv;
  if ((int)blockIdx.x >= a.nch0) {
    kchan_window_chunk(a, blockIdx.x - a.nch0, u, b, hk, qf, reinterpret_cast<float*>(ovB), hm, hl);
    return;
  }
  const int nq = a.counters[b * 4 + 1];
  const BufRes rK = make_res(a.kwords + (size_t)u * a.tiles * 8 * 16, a.tiles * 8 * 16 * 4);
  const BufRes rKM = make_res(a.kmeta + (size_t)u * a.kblocks * kKcKB, a.kblocks * kKcKB * 4);
  const BufRes rS = make_res(a.sparse + (size_t)u * a.cap * a.spv, a.cap * a.spv * 4);
  const BufRes rV = make_res(a.vwords + (size_t)u * a.vrows * kD, a.vrows * kD * 4);
  const BufRes rVM = make_res(a.vmeta + (size_t)u * a.tiles * NG * 16, a.tiles * NG * 16 * 4);
  constexpr int VMETA = VU / 16 * NG * 16 / 64;            // value meta words per lane
  // every word a lane reads for its chunk (out-of-range offsets read 0), in
  // the order it is needed: the vector-memory counter is in order
  struct Chunk {
    uint32_t km[3], sp[kKcTW][2], kw[kKcTW][2], vm[VMETA], vw[8][R];
  };
  auto load_chunk = [&](Chunk& d, int c) {
    const int s0 = c * kKcCH, tile0 = s0 / 16;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int e = tid + 256 * k;
      d.km[k] = e < kKcNB * kKcKB ? bload(rKM, (uint32_t)((s0 / kKcKB) * kKcKB + e) * 4u) : 0u;
    }
    // lanes (n, 0) and (n, 1) score token n: both take its sparse entries
#pragma unroll
    for (int i = 0; i < kKcTW; ++i) {
      const uint32_t tok = (uint32_t)(s0 + 16 * (kKcTW * w + i) + n);
      d.sp[i][0] = d.sp[i][1] = 0u;
      if (j < 2) {
        if (a.spv == 2) {
          const u32x2 e = bload2(rS, tok * 8u);
          d.sp[i][0] = e[0];
          d.sp[i][1] = e[1];
        } else if (a.spv == 1) {
          d.sp[i][0] = bload(rS, tok * 4u);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kKcTW; ++i) {
      const int t = kKcTW * w + i;
#pragma unroll
      for (int x = 0; x < 2; ++x) d.kw[i][x] = bload(rK, (((tile0 + t) * 8 + j + 4 * x) * 16 + n) * 4u);
    }
    const int mt0 = (s0 + VU * w) / 16;
#pragma unroll
    for (int k = 0; k < VMETA; ++k) d.vm[k] = bload(rVM, (uint32_t)(mt0 * NG * 16 + lane + 64 * k) * 4u);
    const int row0 = (s0 + VU * w) / NVV + j * R;
#pragma unroll
    for (int v = 0; v < 8; ++v)
#pragma unroll
      for (int r2 = 0; r2 < R; ++r2) d.vw[v][r2] = bload(rV, ((row0 + r2) * kD + 16 * v + n) * 4u);
  };
  const int c = blockIdx.x;
  float* part = a.part + ((size_t)u * a.nch_total + c) * kGqa * kPartF;
  const int s_begin = c * kKcCH, s_end = min(nq, s_begin + kKcCH);
  if (s_begin >= s_end) {
    for (int i = tid; i < kGqa * kPartF; i += 256) part[i] = (i % kPartF == 0) ? -INFINITY : 0.f;
    return;
  }
  // ---- the query (two channels a thread), then every load of the chunk
  static_assert(kGqa * kD == 2 * 256, "one query word per thread");
  const uint32_t qw =
      reinterpret_cast<const uint32_t*>(a.q + ((size_t)b * a.Hkv * kGqa + hk * kGqa) * kD)[tid];
  Chunk cur;
  load_chunk(cur, c);
  qf[tid / (kD / 2)][2 * (tid % (kD / 2))] = h2f(qw & 0xFFFFu);
  qf[tid / (kD / 2)][2 * (tid % (kD / 2)) + 1] = h2f(qw >> 16);
  DV::fill(ctab, tid, 256);
  const auto& kw = cur.kw;
  const auto& sp = cur.sp;
  const auto& km = cur.km;
  const auto& vw = cur.vw;
  const auto& vm = cur.vm;
#pragma unroll
  for (int k = 0; k < 3; ++k)
    if (tid + 256 * k < kKcNB * kKcKB) kms[tid + 256 * k] = km[k];
  __syncthreads();
  // ---- key-scale operand tables of the chunk's five blocks
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int e = tid + 256 * k;
    if (e < kKcNB * kKcKB) {
      const int blk = e / kKcKB, ch = e % kKcKB;
      const float sg = h2f(km[k] & 0xFFFFu);
      // operand position of channel ch: word jj + 4 (m/2), digit d
      const int word = ch >> 4, d = ch & 15;
      const int tt = d < 8 ? 2 * d : 2 * (d - 8) + 1;      // output index within the word
      const int jj = word & 3, m = 2 * (word >> 2) + (tt >> 3), i = tt & 7;
#pragma unroll
      for (int h = 0; h < kGqa; ++h) {
        const float A = 4.0f * qf[h][ch] * sg;             // exact: two 11-bit significands
        const _Float16 hi = (_Float16)A;
        atab[blk][m][jj][2 * h][i] = hi;
        atab[blk][m][jj][2 * h + 1][i] = (_Float16)(A - (float)hi);
      }
    }
  }
  // sum_d q_h[d] (z_d - 4 s_d) per (block, head): wave w takes pairs w, w + 4, ...;
  // lanes hold channels l and l + 64 (fixed reduction order)
  for (int pr = w; pr < kKcNB * kGqa; pr += 4) {
    const int blk = pr >> 2, h = pr & 3;
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = lane + 64 * k;
      const uint32_t mw = kms[blk * kKcKB + ch];
      o = __builtin_fmaf(qf[h][ch], __builtin_fmaf(-4.0f, h2f(mw & 0xFFFFu), h2f(mw >> 16)), o);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) o += __shfl_xor(o, off);
    if (lane == 0) aoff[blk][h] = o;
  }
  __syncthreads();
  // ---- keys: ten tiles per wave
#pragma unroll
  for (int i = 0; i < kKcTW; ++i) {
    const int t = kKcTW * w + i, blk = t >> 3;
    _Float16 dg[DKc::NOUT];
    DKc::run(kw[i], dg);
    f4 pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      h8 bk, ak;
#pragma unroll
      for (int e = 0; e < 8; ++e) bk[e] = dg[8 * m + e];
      // rows 8..15 repeat rows 0..7: they only reach result rows no lane reads
      ak = *reinterpret_cast<const h8*>(&atab[blk][m][j][n & 7][0]);
      pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(ak, bk, pr, 0, 0, 0);
    }
    // lane (n, j), j < 2: rows 4j..4j+3 = (hi, lo) of heads 2j and 2j + 1,
    // plus the token's sparse entries
    if (j < 2) {
      float x0 = pr[0] + pr[1], x1 = pr[2] + pr[3];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (e < a.spv) {
          const int ch = (int)(sp[i][e] >> 16) & (kD - 1);
          const float val = h2f(sp[i][e] & 0xFFFFu);
          x0 = __builtin_fmaf(qf[2 * j][ch], val, x0);
          x1 = __builtin_fmaf(qf[2 * j + 1][ch], val, x1);
        }
      }
      const bool ok = s_begin + 16 * t + n < s_end;
      sc[2 * j][16 * t + n] = ok ? (x0 + aoff[blk][2 * j]) * a.c : -INFINITY;
      sc[2 * j + 1][16 * t + n] = ok ? (x1 + aoff[blk][2 * j + 1]) * a.c : -INFINITY;
    }
  }
  __syncthreads();
  // ---- softmax over the chunk (wave w: head w) and value meta staging
  // (flagged sequences: value scales enter the fp16 product divided by 2^6)
  const bool vbig = (a.counters[b * 4 + 3] & kFlagBigValueScale) != 0;
  {
    const int h = w;
    float mx = -INFINITY;
    for (int i = lane; i < kKcCH; i += 64) mx = fmaxf(mx, sc[h][i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float l = 0.f;
    for (int i = lane; i < kKcCH; i += 64) {
      const float p = __builtin_amdgcn_exp2f(sc[h][i] - mx);
      l += p;
      const int unit = i / VU, rem = i % VU, jj = rem / (R * NVV), rr = rem % (R * NVV);
      const float xq = __uint_as_float(__float_as_uint(p * kAScale) + 0x1000u);
      pw[h][unit * 4 * VK + jj * VK + DV::pos_of(rr / NVV, rr % NVV)] =
          __builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz(xq, xq))[0];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) { hm[h] = mx; hl[h] = l; }
#pragma unroll
    for (int k = 0; k < VMETA; ++k) {
      const int e = lane + 64 * k;
      const int g = (e % (NG * 16)) / 16, sl = (e / (NG * 16)) * 16 + (e % 16);   // slot in the unit
      const int jj = sl / (R * NVV), rr = sl % (R * NVV);
      const int pos = w * 4 * VK + jj * VK + DV::pos_of(rr / NVV, rr % NVV);
      const bool ok = s_begin + VU * w + sl < s_end;
      vsl[g][pos] = value_scale_operand(ok ? vm[k] : 0u, vbig);
      vzl[g][pos] = __builtin_bit_cast(_Float16, (uint16_t)(ok ? (vm[k] >> 16) : 0u));
    }
  }
  __syncthreads();
  // ---- values: wave w runs unit w
  {
    const int h = n & 3, g = n >> 2;
    float zacc = 0.f;
    h8 av[VM];
#pragma unroll
    for (int m = 0; m < VM; ++m) {
      const int pos = w * 4 * VK + j * VK + 8 * m;
      const h8 p16 = *reinterpret_cast<const h8*>(&pw[h][pos]);
      const h8 sv = *reinterpret_cast<const h8*>(&vsl[g][pos]);
      const h8 zv = *reinterpret_cast<const h8*>(&vzl[g][pos]);
      av[m] = p16 * sv;
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        zacc = __builtin_amdgcn_fdot2((h2v){p16[e], p16[e + 1]}, (h2v){zv[e], zv[e + 1]}, zacc, false);
    }
    f4 acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      acc[v] = (f4){0.f, 0.f, 0.f, 0.f};
      h8 bv[VM];
      DV::run(vw[v], ctab, bv);
#pragma unroll
      for (int m = 0; m < VM; ++m) acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[m], bv[m], acc[v], 0, 0, 0);
    }
    float zs = zacc;
    zs += __shfl_xor(zs, 16);
    zs += __shfl_xor(zs, 32);
    if (lane < 16) zr[w][lane] = zs;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      if ((v >> 1) != j) continue;             // channels 16v..16v+15 are in group v/2
#pragma unroll
      for (int hh = 0; hh < kGqa; ++hh)
        red[w][hh][16 * v + n] = acc[v][hh] * (vbig ? kBigValueShift : 1.0f) + zr[w][4 * j + hh];
    }
  }
  __syncthreads();
  for (int i = tid; i < kGqa * kD; i += 256) {
    const int hh = i / kD, d = i % kD;
    part[hh * kPartF + 4 + d] = (red[0][hh][d] + red[1][hh][d] + red[2][hh][d] + red[3][hh][d]) * (1.0f / kAScale);
  }
  if (tid < kGqa) {
    part[tid * kPartF + 0] = hm[tid];
    part[tid * kPartF + 1] = hl[tid];
  }
}

// Matrix-core decode of the quantized per-channel-key part when its shape
// is the one above (4-level keys, 3-level values, groups of 32, blocks of
// 128, at most two sparse entries); false: not this shape.
bool launch_decode_kchan_mfma(const kvq_layout* L, const uint8_t* cache, const void* q, float c,
                              float* part, int nch0, int nwch, int nch_total, void* stream) {
  const kvq_config& cf = L->cfg;
  if (cf.k_levels != 4 || cf.v_levels != 3 || cf.v_group != 32 || cf.k_block != kKcKB ||
      cf.sparse_per_vec > 2 || L->kw[0] != 8 || decode_chunk_kchan(L) != kKcCH ||
      ((uintptr_t)q & 3) != 0)     // the query is read a word at a time
    return false;
  KchanDecArgs a;
  a.counters = (const int32_t*)(cache + L->counters);
  a.q = (const uint16_t*)q;
  a.part = part;
  a.kwords = (const uint32_t*)(cache + L->k_words[0]);
  a.kmeta = (const uint32_t*)(cache + L->k_meta[0]);
  a.sparse = (const uint32_t*)(cache + L->sparse);
  a.vwords = (const uint32_t*)(cache + L->v_words[0]);
  a.vmeta = (const uint32_t*)(cache + L->v_meta[0]);
  a.Hkv = cf.kv_heads; a.tiles = L->tiles[0]; a.kblocks = L->kblocks; a.vrows = L->vrows[0];
  a.cap = cf.capacity; a.spv = cf.sparse_per_vec; a.nch_total = nch_total;
  a.kwin = (const uint16_t*)(cache + L->k_win);
  a.vwin = (const uint16_t*)(cache + L->v_win);
  a.nch0 = nch0; a.win_cap = L->win_cap;
  a.c = c;
  if (nch0 + nwch > 0)
    k_decode_kchan_mfma<3, 32><<<dim3(nch0 + nwch, cf.batch * cf.kv_heads), 256, 0, (hipStream_t)stream>>>(a);
  return true;
}

}  // namespace kvq
