// Attention of a block of new query tokens over the packed tiered cache, on
// the matrix cores (gfx950 v_mfma_f32_16x16x32_f16).  SemKV, Abstract: the
// quantized history reappears when a conversation continues; every new token
// of the turn reads the whole cache.  Each query row gets its output and its
// log-sum-exp, so that the caller can merge it with attention over the new
// tokens themselves.
//
// Same packed words, operand orders and exact (scale, zero) split as the
// one-query decode kernel; the difference is what fills the 16 rows of the
// matrix instruction: four query tokens x four heads, r = 4 m + h, instead of
// four 32-channel sub-groups x four heads.  The digits of a key tile are
// expanded once; each scale group g multiplies them by the A operands (the
// query at g's channels, zero elsewhere) of just those operand positions
// that carry a channel of g (a compile-time table), built by the key wave in
// registers (read from LDS where there are too many); the value digits of a
// channel tile once, against A = p * s of that tile's sub-group.  So the
// expansion work, the part that bounds one query, is shared by four query
// tokens.
//   keys wave:   lane (n, j) gets rows (j, 0..3) of column n: query j, four
//                heads, slot n; per group it adds s_g * P + z_g * Q_g
//                (Q_g = sum of the query over the group) in fp32;
//                online softmax per row; weights 2^6 p as fp16 into an LDS
//                double buffer, rescale factors alongside.
//   values wave: per macro tile A = p * s per sub-group, column-word digits,
//                matrix ops into the accumulators; sum p z per group on the
//                VALU.
// Partials (m, l, acc) per (unit, query group, chunk, row) are merged by
// k_merge_mq, which also writes the log-sum-exp.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "mfma_util.h"
#include "tiling.h"
#include "unpack.h"

namespace kvq {

constexpr int kMqQ = 4;               // query tokens per workgroup
constexpr int kMqR = kMqQ * kGqa;     // result rows (query, head), r = 4 m + h
constexpr int kMqAqRegsMax = 12;     // key A operands held in registers up to this count

// Key operands per (scale group g, operand mo): lane group jl's elements of
// operand mo are digits of its words jl, jl + 4, ...; the A operand of group
// g is the query at the channels of g among them and zero elsewhere, so the
// matrix op of (g, mo) contributes only where one of those channels falls
// in g.  need[g][mo] marks those; idx numbers them (the A operands kept).
template <class DK, int KW, int NV, int KM, int G>
struct KeyGroupOps {
  static constexpr int NG = kD / G;
  struct Tab {
    bool need[kD / 32][8];
    int idx[kD / 32][8];
    int g_of[32], mo_of[32];
    int n;
  };
  static constexpr Tab make() {
    Tab t{};
    for (int g = 0; g < kD / 32; ++g)
      for (int mo = 0; mo < 8; ++mo) {
        t.need[g][mo] = false;
        t.idx[g][mo] = -1;
      }
    for (int mo = 0; mo < KM; ++mo)
      for (int jl = 0; jl < 4; ++jl) {
        const int nw = (KW - jl + 3) / 4;
        for (int i = 0; i < 8; ++i) {
          const int tt = 8 * mo + i;
          const int wi = DK::word_of(tt);
          if (wi < 0 || wi >= nw) continue;
          const int d = (jl + 4 * wi) * NV + DK::digit_of(tt);
          if (d < kD) t.need[d / G][mo] = true;
        }
      }
    t.n = 0;
    for (int g = 0; g < NG; ++g)
      for (int mo = 0; mo < KM; ++mo)
        if (t.need[g][mo]) {
          t.g_of[t.n] = g;
          t.mo_of[t.n] = mo;
          t.idx[g][mo] = t.n++;
        }
    return t;
  }
  static constexpr Tab kTab = make();
  static_assert(KM <= 8 && kTab.n <= 32, "key operand table");
};

// f(integral_constant<int, i>) for i = B .. E-1, unrolled at compile time
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Waves per SIMD the register allocation aims at: two, except the 5-level
// grid with 64-channel groups, whose two waves would need about 270
// registers (it spills at 256) and which takes one.
__host__ __device__ constexpr int mq_min_waves(int L, int G) { return (L == 5 && G == 64) ? 1 : 2; }

template <int L, int G>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(mq_min_waves(L, G)))) void k_decode_pool_mq(
    PoolMqArgs a) {
  using T = Tiling<L>;
  constexpr int NV = T::NV, KW = T::KW, KWL = T::KWL, R = T::R, RUN = T::RUN, MT = T::MT,
                KT = T::KT;
  using DK = Unpack<L, KWL>;
  using DV = Unpack<L, R>;
  constexpr int KM = DK::NH8, VM = DV::NH8;
  constexpr bool AFF = DK::kAffine;
  constexpr float MUL = (float)DK::kMul;
  constexpr int NG = kD / G;                 // (scale, zero) groups per row
  constexpr int NS = kD / 32;                // 32-channel sub-groups per row
  constexpr int SUB = G / 32;                // sub-groups per group
  constexpr int VK = VM * 8;                 // padded slot run per lane group
  constexpr int META = KT * NG * 16;         // (scale, zero) words per macro tile
  constexpr int META_PER_LANE = (META + 63) / 64;
  using KG = KeyGroupOps<DK, KW, NV, KM, G>;
  constexpr int NA = KG::kTab.n;             // key A operands (group, operand) kept

  // the key A operands stay in registers when they fit beside the rest
  constexpr bool kAqRegs = NA <= kMqAqRegsMax;
  // The query rows are read only during set-up and the weights only after
  // it, so they share LDS; the key wave builds its A operands in registers
  // straight from the rows (a 5-level workgroup takes 33 KB, four per CU; a
  // 6-level one 22 KB, six).
  union SetupOrPw {
    struct {
      _Float16 qh[kMqR][kD];                 // query rows (fp16, as given)
    } s;
    _Float16 pw[2][kMqR][4 * VK];            // 2^6 p, operand order
    uint4 raw[2 * kMqR * 4 * VK * 2 / 16];   // the weights as 16-byte words
  };
  __shared__ __attribute__((aligned(16))) SetupOrPw sp;
  __shared__ h8 aq_keep[kAqRegs ? 1 : NA][64];   // key A operands kept in LDS
  __shared__ float qcs[NG][kMqR];            // c * sum of row r's query over group g
  constexpr int kPwBytes = 2 * kMqR * 4 * VK * 2;
  __shared__ uint32_t km_lds[META_PER_LANE * 64];   // key (scale, zero) of the macro tile
  __shared__ float al_lds[2][kMqR];          // rescale factor per row
  __shared__ __attribute__((aligned(16))) _Float16 vs_lds[NG][4 * VK];  // value scale
  __shared__ __attribute__((aligned(16))) _Float16 vz_lds[NG][4 * VK];  // value zero
  __shared__ int ppos_lds[MT];               // slot -> operand position
  __shared__ int mpos_lds[64 * META_PER_LANE];
  __shared__ float zred[NG][kMqR];
  __shared__ uint2 ctab[DK::kTableEntries];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const int c = blockIdx.x, u = blockIdx.y, qg = blockIdx.z;
  const int b = u / a.Hkv, hk = u % a.Hkv;
  float* part = a.part + (((size_t)u * a.nqg + qg) * a.nch_total + a.part_off + c) * kMqR * kPartF;
  const int n_valid = a.counters[b * 4 + 1 + a.pool];
  // the unit's filled slots split evenly over the launch's chunks, in whole
  // macro tiles (the grid is sized for the pool's capacity, which can exceed
  // the filled slots by a whole chunk's share)
  const int span = ((n_valid + MT - 1) / MT + (int)gridDim.x - 1) / (int)gridDim.x * MT;
  const int s_begin = c * span;
  const int s_end = min(n_valid, s_begin + span);
  if (s_begin >= s_end) {
    for (int i = threadIdx.x; i < kMqR * kPartF; i += 128) part[i] = (i % kPartF == 0) ? -INFINITY : 0.f;
    return;
  }
  const int nmt = (s_end - s_begin + MT - 1) / MT;

  // ---- shared set-up: query rows (absent queries are zero), operand maps
  const int Hq = a.Hkv * kGqa;
  for (int i = threadIdx.x; i < kMqR * kD; i += 128) {
    const int r = i / kD, d = i % kD, m = qg * kMqQ + (r >> 2);
    const int src = a.korder ? (int)(a.korder[(size_t)hk * kD + d] & 0x7F) : d;   // stored order
    sp.s.qh[r][d] = __builtin_bit_cast(
        _Float16, (uint16_t)(m < a.M ? a.q[(((size_t)b * a.M + m) * Hq + hk * kGqa + (r & 3)) * kD + src] : 0));
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
  for (int i = threadIdx.x; i < 4 * VK; i += 128)
    for (int g = 0; g < NG; ++g) { vs_lds[g][i] = (_Float16)0.0f; vz_lds[g][i] = (_Float16)0.0f; }
  __syncthreads();
  // key A operands: lane (row n, k-block jl) of operand (g, mo) holds the
  // query of row n at the channels of group g its operand positions carry,
  // zero elsewhere (here only when they stay in LDS)
  if constexpr (!kAqRegs) {
    for (int e = threadIdx.x; e < NA * 64; e += 128) {
      const int ai = e / 64, l = e % 64;
      const int gq = KG::kTab.g_of[ai], mo = KG::kTab.mo_of[ai];
      const int rn = l & 15, jl = l >> 4;
      const int nw = (KW - jl + 3) / 4;        // words lane group jl owns
      h8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 8 * mo + i;
        const int wi = DK::word_of(t);
        const int d = (jl + 4 * wi) * NV + DK::digit_of(t);
        const bool ok = wi >= 0 && wi < nw && d < kD && d / G == gq;
        v[i] = ok ? sp.s.qh[rn][min(max(d, 0), kD - 1)] : (_Float16)0.0f;
      }
      aq_keep[ai][l] = v;
    }
  }
  for (int e = threadIdx.x; e < NG * kMqR; e += 128) {
    const int g = e / kMqR, r = e % kMqR;
    float sum = 0.f;
    for (int d = 0; d < G; ++d) sum += (float)sp.s.qh[r][G * g + d];
    qcs[g][r] = sum * a.c;
  }
  __syncthreads();

  if (wave == 0) {
    // the key chain sets the pace of the pair: it issues first on its SIMD
    __builtin_amdgcn_s_setprio(3);
    // ================= keys: scores, softmax, weights =================
    const BufRes rK = make_res(a.kwords + (size_t)u * a.tiles * KW * 16, a.tiles * KW * 16 * 4);
    const BufRes rKM = make_res(a.kmeta + (size_t)u * a.tiles * NG * 16, a.tiles * NG * 16 * 4);
    uint32_t kwoff[KWL];
#pragma unroll
    for (int wi = 0; wi < KWL; ++wi) {
      const int w = j + 4 * wi;
      kwoff[wi] = w < KW ? (uint32_t)(w * 16 + n) * 4u : kOutOfRange;
    }
    struct KBuf {
      uint32_t kw[KT][KWL];
      uint32_t km[META_PER_LANE];
    };
    auto load_k = [&](KBuf& kb, int s0) {
      const uint32_t tile0 = s0 / 16;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int wi = 0; wi < KWL; ++wi) kb.kw[t][wi] = bload(rK, kwoff[wi] + (tile0 + t) * (KW * 16 * 4));
#pragma unroll
      for (int k = 0; k < META_PER_LANE; ++k) {
        const int e = lane + 64 * k;
        kb.km[k] = bload(rKM, (META % 64 == 0 || e < META) ? (tile0 * NG * 16 + e) * 4u : kOutOfRange);
      }
    };
    KBuf nxt;
    load_k(nxt, s_begin);
    float qc[NG][kGqa];                      // c * sum over group g of row (j, h)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int h = 0; h < kGqa; ++h) qc[g][h] = qcs[g][4 * j + h];
    int spos[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) spos[t] = ppos_lds[16 * t + n];
    h8 aqr[kAqRegs ? NA : 1];
    if constexpr (kAqRegs) {
      const int nwj = (KW - j + 3) / 4;      // words lane group j owns
      static_for<0, NA>([&](auto ac) __attribute__((always_inline)) {
        constexpr int ai = decltype(ac)::value;
        constexpr int gq = KG::kTab.g_of[ai], mo = KG::kTab.mo_of[ai];
        h8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t = 8 * mo + i;
          const int wi = DK::word_of(t);
          const int d = (j + 4 * wi) * NV + DK::digit_of(t);
          const bool ok = wi >= 0 && wi < nwj && d < kD && d / G == gq;
          v[i] = ok ? sp.s.qh[n][min(max(d, 0), kD - 1)] : (_Float16)0.0f;
        }
        aqr[ai] = v;
      });
    }
    // set-up data read: clear the weight buffers that share its LDS (operand
    // positions no slot fills stay zero); the other wave reads them only
    // after the first macro tile's barrier
    wave_lds_fence();
    for (int i = lane; i < kPwBytes / 16; i += 64) sp.raw[i] = make_uint4(0u, 0u, 0u, 0u);
    float m_run[kGqa], l_run[kGqa];
#pragma unroll
    for (int h = 0; h < kGqa; ++h) { m_run[h] = -INFINITY; l_run[h] = 0.f; }
    for (int it = 0; it <= nmt; ++it) {
      if (it < nmt) {
        const int s0 = s_begin + it * MT;
        const KBuf cur = nxt;
        if (it + 1 < nmt) load_k(nxt, s0 + MT);
        // this macro tile's key (scale, zero), [tile][group][slot]; only this
        // wave uses km_lds and its LDS accesses execute in order
#pragma unroll
        for (int k = 0; k < META_PER_LANE; ++k) km_lds[lane + 64 * k] = cur.km[k];
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        float scs[KT][kGqa];
        float mx[kGqa];
#pragma unroll
        for (int h = 0; h < kGqa; ++h) mx[h] = -INFINITY;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          h8 bk[KM];
          DK::run(cur.kw[t], ctab, bk);
          float x[kGqa] = {0.f, 0.f, 0.f, 0.f};
          static_for<0, NG>([&](auto gc) __attribute__((always_inline)) {
            constexpr int g = decltype(gc)::value;
            f4 pr = {0.f, 0.f, 0.f, 0.f};
            static_for<0, KM>([&](auto mc) __attribute__((always_inline)) {
              constexpr int mo = decltype(mc)::value;
              constexpr int ai = KG::kTab.idx[g][mo];
              if constexpr (ai >= 0)
                pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(kAqRegs ? aqr[kAqRegs ? ai : 0] : aq_keep[kAqRegs ? 0 : ai][lane],
                                                            bk[mo], pr, 0, 0, 0);
            });
            const uint32_t meta = km_lds[(t * NG + g) * 16 + n];
            const float sgf = h2f(meta & 0xFFFFu) * MUL;
            const float ssc = sgf * a.c, zz = AFF ? h2f(meta >> 16) - sgf : h2f(meta >> 16);
#pragma unroll
            for (int h = 0; h < kGqa; ++h) x[h] = __builtin_fmaf(ssc, pr[h], __builtin_fmaf(zz, qc[g][h], x[h]));
          });
          const bool ok = s0 + 16 * t + n < s_end;
#pragma unroll
          for (int h = 0; h < kGqa; ++h) {
            scs[t][h] = ok ? x[h] : -INFINITY;
            mx[h] = fmaxf(mx[h], scs[t][h]);
          }
        }
        // online softmax of rows (j, h); weights as fp16 2^6 p, formed by one
        // exp2 with the 2^6 folded into the max and rounded to nearest even
        // (unbiased, as the one-query kernel's half-up rounding)
#pragma unroll
        for (int h = 0; h < kGqa; ++h) {
          const float m_new = fmaxf(m_run[h], row_max16(mx[h]));
          const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_use);
          const float m6 = m_use - 6.0f;     // 2^6 p = exp2(s - (m - 6))
          _Float16* pb = &sp.pw[it & 1][4 * j + h][0];
          float ls = 0.f;                    // in units of 2^-6
#pragma unroll
          for (int t = 0; t < KT; ++t) {
            const float p6 = __builtin_amdgcn_exp2f(scs[t][h] - m6);
            ls += p6;
            pb[spos[t]] = (_Float16)p6;     // round to nearest even
          }
          l_run[h] = __builtin_fmaf(l_run[h], alpha, ls);
          m_run[h] = m_new;
          if (n == 0) al_lds[it & 1][4 * j + h] = alpha;
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int h = 0; h < kGqa; ++h) {
      const float l_tot = row_sum16(l_run[h]);
      if (n == 0) {
        part[(4 * j + h) * kPartF + 0] = m_run[h];
        part[(4 * j + h) * kPartF + 1] = l_tot * (1.0f / kAScale);
      }
    }
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
    // flagged sequences: value scales enter the fp16 product divided by 2^6
    const bool vbig = (a.counters[b * 4 + 3] & kFlagBigValueScale) != 0;
    // A-operand view: lane (n, j) holds row n = (query n / 4, head n % 4)
    // over the operand positions of lane group j
    float zacc[NG];                          // 2^6 sum p z per group (row n)
#pragma unroll
    for (int g = 0; g < NG; ++g) zacc[g] = 0.f;
    f4 acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = (f4){0.f, 0.f, 0.f, 0.f};
    f4 asum[NS];                             // power-of-two grids: sum of A per row and sub-group
#pragma unroll
    for (int sg = 0; sg < NS; ++sg) asum[sg] = (f4){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it <= nmt; ++it) {
      if (it >= 1) {
        const int i = it - 1;
        const int s0 = s_begin + i * MT;
        const VBuf cur = nxt;
        if (i + 1 < nmt) load_v(nxt, s0 + MT);
        float al[kGqa];
#pragma unroll
        for (int hh = 0; hh < kGqa; ++hh) al[hh] = al_lds[i & 1][4 * j + hh];
        const float aln = al_lds[i & 1][n];
        // accumulator rows are (query j, head = register index)
#pragma unroll
        for (int v = 0; v < 8; ++v)
#pragma unroll
          for (int hh = 0; hh < kGqa; ++hh) acc[v][hh] *= al[hh];
        if (AFF)
#pragma unroll
          for (int sg = 0; sg < NS; ++sg)
#pragma unroll
            for (int hh = 0; hh < kGqa; ++hh) asum[sg][hh] *= al[hh];
#pragma unroll
        for (int g = 0; g < NG; ++g) zacc[g] *= aln;
        // value (scale, zero) in operand order (only this wave uses vs/vz)
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
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        // zero-point sums
#pragma unroll
        for (int m = 0; m < VM; ++m) {
          const int pos = j * VK + 8 * m;
          const h8 p16 = *reinterpret_cast<const h8*>(&sp.pw[i & 1][n][pos]);
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const h8 zv = *reinterpret_cast<const h8*>(&vz_lds[g][pos]);
#pragma unroll
            for (int e = 0; e < 8; e += 2)
              zacc[g] = __builtin_amdgcn_fdot2((h2v){p16[e], p16[e + 1]}, (h2v){zv[e], zv[e + 1]}, zacc[g], false);
          }
        }
        // channel tiles v = 2 sg, 2 sg + 1 share the A operand of sub-group sg
#pragma unroll
        for (int sg = 0; sg < NS; ++sg) {
          const int g = sg / SUB;
          h8 av[VM];
#pragma unroll
          for (int m = 0; m < VM; ++m) {
            const int pos = j * VK + 8 * m;
            const h8 p16 = *reinterpret_cast<const h8*>(&sp.pw[i & 1][n][pos]);
            const h8 sv = *reinterpret_cast<const h8*>(&vs_lds[g][pos]);
            av[m] = p16 * sv;                // fp16 products, rounded to nearest
          }
          if (AFF) {
            const h8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
            for (int m = 0; m < VM; ++m) asum[sg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[m], ones, asum[sg], 0, 0, 0);
          }
#pragma unroll
          for (int vv = 0; vv < 2; ++vv) {
            const int v = 2 * sg + vv;
            h8 bv[VM];
            DV::run(cur.vw[v], ctab, bv);
#pragma unroll
            for (int m = 0; m < VM; ++m) acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[m], bv[m], acc[v], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }
    // partials.  zacc: lanes (n, j) -> sum over j per row n and group.
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float zs = zacc[g];
      zs += __shfl_xor(zs, 16);
      zs += __shfl_xor(zs, 32);
      if (lane < 16) zred[g][lane] = zs;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // power-of-two grids: digits are 1 + d/MUL, so sum p s d = MUL (acc - asum)
    const float vfac = MUL * (vbig ? kBigValueShift : 1.0f);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int sg = v >> 1, g = sg / SUB, d = 16 * v + n;
#pragma unroll
      for (int hh = 0; hh < kGqa; ++hh) {
        const float t = (acc[v][hh] - (AFF ? asum[sg][hh] : 0.f)) * vfac + zred[g][4 * j + hh];
        part[(4 * j + hh) * kPartF + 4 + d] = t * (1.0f / kAScale);
      }
    }
  }
}

// Log-sum-exp merge over every chunk of both pools: workgroup = (unit,
// query group, row), thread = channel.  Chunks are read kMqBatch at a time
// (one memory round trip per batch) into a running maximum, rescaling what
// has been summed when it grows.  Output fp16 [B][M][Hq][D]; lse (natural
// log, scores scaled) [B][M][Hq] when given.
constexpr int kMqBatch = 8;
__global__ __launch_bounds__(kD) void k_merge_mq(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                float* __restrict__ lse, int nch, int nqg, int M, int Hkv,
                                                const uint8_t* __restrict__ vorder) {
  const int row = blockIdx.x, r = row % kMqR, ug = row / kMqR;
  const int qg = ug % nqg, u = ug / nqg;
  const int m = qg * kMqQ + (r >> 2);
  if (m >= M) return;
  const int h = r & 3, b = u / Hkv, hk = u % Hkv, d = threadIdx.x;
  const float* base = part + (size_t)ug * nch * kMqR * kPartF + r * kPartF;
  constexpr int kStep = kMqR * kPartF;
  float mx = -INFINITY, l = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nch; c0 += kMqBatch) {
    float mc[kMqBatch], lc[kMqBatch], ac[kMqBatch];
#pragma unroll
    for (int k = 0; k < kMqBatch; ++k) {
      const bool ok = c0 + k < nch;
      const float* p = base + (size_t)(ok ? c0 + k : c0) * kStep;
      mc[k] = ok ? p[0] : -INFINITY;
      lc[k] = ok ? p[1] : 0.f;
      ac[k] = ok ? p[4 + d] : 0.f;
    }
    float bm = mx;
#pragma unroll
    for (int k = 0; k < kMqBatch; ++k) bm = fmaxf(bm, mc[k]);
    if (bm == -INFINITY) continue;
    const float f = __builtin_amdgcn_exp2f(mx - bm);      // 0 while nothing has been summed
    l *= f;
    acc *= f;
#pragma unroll
    for (int k = 0; k < kMqBatch; ++k) {
      const float w = __builtin_amdgcn_exp2f(mc[k] - bm);  // 0 for empty chunks
      l = __builtin_fmaf(w, lc[k], l);
      acc = __builtin_fmaf(w, ac[k], acc);
    }
    mx = bm;
  }
  const size_t o = ((size_t)b * M + m) * Hkv * kGqa + hk * kGqa + h;
  // position d of the sums is channel vorder[d] of the output (stored order)
  out[o * kD + (vorder ? (int)(vorder[(size_t)hk * kD + d] & 0x7F) : d)] = (uint16_t)f2h_rne(acc / l);
  if (lse && d == 0) lse[o] = (mx + __log2f(l)) * 0.69314718055994530942f;
}

template <int L, int G>
static void launch_mq_one(const PoolMqArgs& a, int nch, int U, hipStream_t s) {
  k_decode_pool_mq<L, G><<<dim3(nch, U, a.nqg), 128, 0, s>>>(a);
}

template <int L>
static bool launch_mq_L(const PoolMqArgs& a, int G, int nch, int U, hipStream_t s) {
  switch (G) {
    case 32: launch_mq_one<L, 32>(a, nch, U, s); return true;
    case 64: launch_mq_one<L, 64>(a, nch, U, s); return true;
    case 128: launch_mq_one<L, 128>(a, nch, U, s); return true;
  }
  return false;
}

template <int L>
static int mq_occupancy_L(int G) {
  int blocks = 0;
  hipError_t e = hipErrorInvalidValue;
  switch (G) {
    case 32: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pool_mq<L, 32>, 128, 0); break;
    case 64: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pool_mq<L, 64>, 128, 0); break;
    case 128: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k_decode_pool_mq<L, 128>, 128, 0); break;
  }
  return e == hipSuccess ? blocks : 0;
}

// Workgroups per CU of the multi-query pool kernel, cached per device (value
// + 1; 0: not read yet; threads racing on a first read store the same value).
constexpr int kMqMaxDevices = 64;
static std::atomic<int> g_mq_occ[kMqMaxDevices][9][3];

static int mq_occupancy(int L, int G) {
  const int gi = G == 32 ? 0 : G == 64 ? 1 : 2;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const bool cached = dev >= 0 && dev < kMqMaxDevices && L >= 0 && L <= 8;
  int occ = cached ? g_mq_occ[dev][L][gi].load(std::memory_order_relaxed) - 1 : -1;
  if (occ >= 0) return occ;
  switch (L) {
    case 3: occ = mq_occupancy_L<3>(G); break;
    case 4: occ = mq_occupancy_L<4>(G); break;
    case 5: occ = mq_occupancy_L<5>(G); break;
    case 6: occ = mq_occupancy_L<6>(G); break;
    case 7: occ = mq_occupancy_L<7>(G); break;
    case 8: occ = mq_occupancy_L<8>(G); break;
    default: occ = 0;
  }
  if (cached) g_mq_occ[dev][L][gi].store(occ + 1, std::memory_order_relaxed);
  return occ;
}

static bool launch_mq_pool(int L, const PoolMqArgs& a, int G, int nch, int U, hipStream_t s) {
  switch (L) {
    case 3: return launch_mq_L<3>(a, G, nch, U, s);
    case 4: return launch_mq_L<4>(a, G, nch, U, s);
    case 5: return launch_mq_L<5>(a, G, nch, U, s);
    case 6: return launch_mq_L<6>(a, G, nch, U, s);
    case 7: return launch_mq_L<7>(a, G, nch, U, s);
    case 8: return launch_mq_L<8>(a, G, nch, U, s);
  }
  return false;
}

kvq_status launch_decode_mq(const kvq_layout* L, const uint8_t* cache, const void* q, int M, float scale,
                            int max_len, void* out, float* lse, uint8_t* ws, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const kvq_config& c = L->cfg;
  if (c.mode != KVQ_MODE_TIERED) return KVQ_ERR_UNSUPPORTED;
  const int U = c.batch * c.kv_heads, nqg = (M + kMqQ - 1) / kMqQ;
  int nch0, nch1;
  const int nch = decode_chunks(L, max_len, &nch0, &nch1);
  const int lv[2] = {c.levels_hi, c.levels_lo};
  int chunk[2], nchp[2];
  for (int p = 0; p < 2; ++p) {
    const int slots = L->cap[p] < max_len ? L->cap[p] : max_len;
    chunk[p] = chunk_for_one_round(lv[p], U * nqg, slots, mq_occupancy(lv[p], c.group));
    nchp[p] = ceil_div(slots, chunk[p]);
  }
  const int nch_used = nchp[0] + nchp[1];
  if (nch_used > nch) return KVQ_ERR_WORKSPACE;   // the workspace holds the finest split
  const uint8_t* korder = c.reorder ? cache + L->chan_order : nullptr;
  const uint8_t* vorder = c.reorder ? korder + (size_t)c.kv_heads * kD : nullptr;
  for (int p = 0; p < 2; ++p) {
    PoolMqArgs pa;
    pa.counters = (const int32_t*)(cache + L->counters);
    pa.q = (const uint16_t*)q;
    pa.korder = korder;
    pa.part = (float*)ws;
    pa.kwords = (const uint32_t*)(cache + L->k_words[p]);
    pa.kmeta = (const uint32_t*)(cache + L->k_meta[p]);
    pa.vwords = (const uint32_t*)(cache + L->v_words[p]);
    pa.vmeta = (const uint32_t*)(cache + L->v_meta[p]);
    pa.pool = p;
    pa.Hkv = c.kv_heads;
    pa.M = M;
    pa.nqg = nqg;
    pa.tiles = L->tiles[p];
    pa.vrows = L->vrows[p];
    pa.nch_total = nch_used;
    pa.part_off = p ? nchp[0] : 0;
    pa.chunk = chunk[p];
    pa.c = scale * 1.4426950408889634f;
    if (nchp[p] > 0 && !launch_mq_pool(lv[p], pa, c.group, nchp[p], U, s)) return KVQ_ERR_LAUNCH;
  }
  k_merge_mq<<<U * nqg * kMqR, kD, 0, s>>>((const float*)ws, (uint16_t*)out, lse, nch_used, nqg, M,
                                           c.kv_heads, vorder);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH;
}

size_t decode_mq_ws_bytes(const kvq_layout* L, int M, int max_len) {
  int a, b;
  const int n = decode_chunks(L, max_len, &a, &b);
  const size_t U = (size_t)L->cfg.batch * L->cfg.kv_heads, nqg = (M + kMqQ - 1) / kMqQ;
  return U * nqg * (size_t)n * kMqR * kPartF * 4;
}

}  // namespace kvq
