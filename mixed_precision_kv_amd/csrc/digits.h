// Base-L digits of packed words as fp16 matrix operands.
//
// Precondition for the non-power-of-two grids: the wave's fp16/fp64 rounding
// mode is round-toward-zero (set_f16_round_toward_zero()).  Then, for a chunk
// value 0 <= x < L^(j+1) held exactly in fp16,
//   fma(x, c_j, 1024) = 1024 + floor(x / L^j)      with c_j = RU16(1 / L^j),
// because the exact sum lies in [1024, 2048) where the fp16 spacing is 1 and
// truncation is floor; c_j >= 1/L^j keeps exact multiples from falling below
// the integer and (c_j - 1/L^j) * x < 1/L^j keeps the fraction below one
// (checked exhaustively for every chunk value of the supported grids).  The
// digit is that sum minus 1024, and x - L^j * digit is the exact remainder.
// Two chunks ride in the two halves of a packed fp16 register, so each step
// yields two digits for three packed instructions.
//
// Words are first split into chunks that fit fp16 exactly (L^k <= 2048):
// the 32-bit word converts exactly to fp64, floor(x * RU64(1/L^k)) and an fma
// remainder are exact there (also under round-toward-zero), and the parts
// below 2^24 continue in fp32 (round-to-nearest, which is untouched).
//
// Power-of-two grids need no arithmetic: a digit field is or-ed into the
// mantissa of fp16 1.0, giving the affine value 1 + d/M (M = 4 or 8); the
// kernel folds the affine map into the group's (scale, zero).
#pragma once
#include <stdint.h>

#include <type_traits>

#include "tiling.h"

namespace kvq {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// fp16 bits of the smallest fp16 >= 1/N (normal range), by exact integer math.
__host__ __device__ constexpr uint16_t fp16_ru_recip_bits(uint32_t N) {
  // find E with 2^E <= 1/N < 2^(E+1): E = -ceil(log2 N)
  int lg = 0;
  while ((1u << lg) < N) ++lg;            // lg = ceil(log2 N)
  int E = -lg;
  // mantissa M = ceil(2^(10-E) / N) in [1024, 2048]
  uint64_t num = 1ull << (10 - E);
  uint64_t M = (num + N - 1) / N;
  if (M >= 2048) { M = (M + 1) / 2; ++E; }
  return (uint16_t)(((E + 15) << 10) | (M - 1024));
}

__device__ inline h2v h2_splat_bits(uint16_t b) {
  const _Float16 v = __builtin_bit_cast(_Float16, b);
  return (h2v){v, v};
}
__device__ inline h2v h2_splat(float f) {
  const _Float16 v = (_Float16)f;
  return (h2v){v, v};
}
__device__ inline h2v h2_from_bits(uint32_t b) { return __builtin_bit_cast(h2v, b); }
__device__ inline h2v pk_fma(h2v a, h2v b, h2v c) { return __builtin_elementwise_fma(a, b, c); }

__device__ inline void set_f16_round_toward_zero() {
  // MODE.FP_ROUND[3:2] (fp64 and fp16) = 3 (toward zero); fp32 keeps nearest-even.
  asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 2, 2), 3\n\ts_nop 1" ::: "memory");
}

__host__ __device__ constexpr uint32_t ipow(uint32_t L, int k) {
  uint32_t p = 1;
  for (int i = 0; i < k; ++i) p *= L;
  return p;
}

// K digits of each half of x (< L^K), most significant first:
// out[2*i] / out[2*i+1] = digit K-1-i of the low / high half.
template <int L, int K>
__device__ inline void chunk_pair_digits(h2v x, _Float16* out) {
  const h2v k1024 = h2_splat(1024.0f), n1024 = h2_splat(-1024.0f);
#pragma unroll
  for (int j = K - 1; j >= 1; --j) {
    const h2v c = h2_splat_bits(fp16_ru_recip_bits(ipow(L, j)));
    const h2v r = pk_fma(x, c, k1024);
    const h2v d = r + n1024;
    x = pk_fma(d, h2_splat(-(float)ipow(L, j)), x);
    out[2 * (K - 1 - j)] = d[0];
    out[2 * (K - 1 - j) + 1] = d[1];
  }
  out[2 * (K - 1)] = x[0];
  out[2 * (K - 1) + 1] = x[1];
}

__host__ __device__ constexpr double ru64_recip(uint32_t N) { return (1.0 / (double)N) * (1.0 + 0x1p-40); }
__host__ __device__ constexpr float ru32_recip(uint32_t N) {
  return (float)((1.0 / (double)N) * (1.0 + 0x1p-23));
}

// Exact floor(x / N) and remainder of a non-negative integer-valued double.
__device__ inline void split64(double x, uint32_t N, double& q, double& r) {
  q = __builtin_floor(x * ru64_recip(N));
  r = __builtin_fma(q, -(double)N, x);
}
// Same in fp32 for integer values x < 2^24 with x * 2^-22 / N well below 1/N
// (the reciprocal's excess times x stays under the spacing 1/N).
__device__ inline void split32(float x, uint32_t N, float& q, float& r) {
  q = __builtin_floorf(x * ru32_recip(N));
  r = __builtin_fmaf(q, -(float)N, x);
}

// Extraction of NW words of L levels into fp16 values.  Output element t
// holds digit digit_of(t) of word word_of(t) (or is padding, word_of < 0).
template <int L, int NW, class Enable = void>
struct Digits;

// ---- L = 5, 6: chunks of 4 digits (L^4 = 625 / 1296 < 2048) ----
template <int L, int NW>
struct Digits<L, NW, typename std::enable_if<(L == 5 || L == 6)>::type> {
  static constexpr int NV = cpw(L);                    // 13 or 12
  static constexpr bool kAffine = false;
  static constexpr int kMul = 1;
  static constexpr int NAB = NW;                       // (a, b) pairs, one per word
  static constexpr int NC = (NW + 1) / 2;              // (c, c) pairs
  static constexpr int NE = (L == 5) ? (NW + 7) / 8 : 0;   // 8-slot groups of single digits
  static constexpr int NOUT = 8 * (NAB + NC + NE);
  // element t -> (word, digit)
  static constexpr int word_of(int t) {
    if (t < 8 * NAB) return t / 8;
    t -= 8 * NAB;
    if (t < 8 * NC) {
      const int w = 2 * (t / 8) + (t % 2);
      return w < NW ? w : -1;
    }
    t -= 8 * NC;
    return t < NW ? t : -1;
  }
  static constexpr int digit_of(int t) {
    if (t < 8 * NAB) {
      const int i = t % 8;                             // [a3 b3 a2 b2 a1 b1 a0 b0]
      return (3 - i / 2) + ((i % 2) ? 4 : 0);
    }
    t -= 8 * NAB;
    if (t < 8 * NC) return 8 + (3 - (t % 8) / 2);
    return 12;
  }
  __device__ static inline void run(const uint32_t (&w)[NW], _Float16 (&out)[NOUT]) {
    float a[NW], b[NW], c[NW], e[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const double x = (double)w[i];
      double qe, r, qc, r2;
      if (L == 5) {
        split64(x, ipow(5, 12), qe, r);                // top digit 12
        split64(r, ipow(5, 8), qc, r2);
      } else {
        qe = 0.0;
        split64(x, ipow(6, 8), qc, r2);
      }
      float qb, ra;
      split32((float)r2, ipow(L, 4), qb, ra);
      a[i] = ra; b[i] = qb; c[i] = (float)qc; e[i] = (float)qe;
    }
#pragma unroll
    for (int i = 0; i < NAB; ++i)
      chunk_pair_digits<L, 4>(__builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz(a[i], b[i])), &out[8 * i]);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const float hi = (2 * i + 1 < NW) ? c[2 * i + 1] : 0.0f;
      chunk_pair_digits<L, 4>(__builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz(c[2 * i], hi)),
                              &out[8 * NAB + 8 * i]);
    }
#pragma unroll
    for (int t = 0; t < 8 * NE; t += 2) {
      const float lo = t < NW ? e[t] : 0.0f, hi = t + 1 < NW ? e[t + 1] : 0.0f;
      const h2v v = __builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      out[8 * (NAB + NC) + t] = v[0];
      out[8 * (NAB + NC) + t + 1] = v[1];
    }
  }
};

// ---- L = 3: 20 digits as four chunks of 5 (3^5 = 243) ----
template <int NW>
struct Digits<3, NW, void> {
  static constexpr int NV = 20;
  static constexpr bool kAffine = false;
  static constexpr int kMul = 1;
  static constexpr int NOUT = ((20 * NW + 7) / 8) * 8;
  static constexpr int word_of(int t) { return t < 20 * NW ? t / 20 : -1; }
  static constexpr int digit_of(int t) {
    // per word: pair (d0-4, d5-9) then (d10-14, d15-19), each [lo4 hi4 lo3 hi3 ... lo0 hi0]
    const int i = t % 20, p = i / 10, k = i % 10;
    return 10 * p + (4 - k / 2) + ((k % 2) ? 5 : 0);
  }
  __device__ static inline void run(const uint32_t (&w)[NW], _Float16 (&out)[NOUT]) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      double qa, r, qb, r2;
      split64((double)w[i], ipow(3, 15), qa, r);       // qa: digits 15-19
      split64(r, ipow(3, 10), qb, r2);                 // qb: digits 10-14
      float qc, r3;
      split32((float)r2, ipow(3, 5), qc, r3);          // qc: digits 5-9, r3: digits 0-4
      chunk_pair_digits<3, 5>(__builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz(r3, qc)), &out[20 * i]);
      chunk_pair_digits<3, 5>(__builtin_bit_cast(h2v, __builtin_amdgcn_cvt_pkrtz((float)qb, (float)qa)),
                              &out[20 * i + 10]);
    }
#pragma unroll
    for (int t = 20 * NW; t < NOUT; ++t) out[t] = (_Float16)0.0f;
  }
};

// ---- L = 4: 2-bit fields, digits (k, k+8) share a register ----
template <int NW>
struct Digits<4, NW, void> {
  static constexpr int NV = 16;
  static constexpr bool kAffine = true;
  static constexpr int kMul = 4;                       // value = 1 + d/4
  static constexpr int NOUT = 16 * NW;
  static constexpr int word_of(int t) { return t / 16; }
  static constexpr int digit_of(int t) { return (t % 16) / 2 + ((t % 2) ? 8 : 0); }
  __device__ static inline void run(const uint32_t (&w)[NW], _Float16 (&out)[NOUT]) {
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t s = k <= 4 ? (w[i] << (8 - 2 * k)) : (w[i] >> (2 * k - 8));
        const h2v v = h2_from_bits((s & 0x03000300u) | 0x3C003C00u);
        out[16 * i + 2 * k] = v[0];
        out[16 * i + 2 * k + 1] = v[1];
      }
  }
};

// ---- L = 8: 3-bit fields; the high 16 digits' bits are realigned so digits
// (k, k+5) share a register ----
template <int NW>
struct Digits<8, NW, void> {
  static constexpr int NV = 10;
  static constexpr bool kAffine = true;
  static constexpr int kMul = 8;                       // value = 1 + d/8
  static constexpr int NOUT = ((10 * NW + 7) / 8) * 8;
  static constexpr int word_of(int t) { return t < 10 * NW ? t / 10 : -1; }
  static constexpr int digit_of(int t) { return (t % 10) / 2 + ((t % 2) ? 5 : 0); }
  __device__ static inline void run(const uint32_t (&w)[NW], _Float16 (&out)[NOUT]) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      // low half: bits 0..15 of w (digits 0..4); high half: bits 15..30 (digits 5..9)
      const uint32_t hi = __builtin_amdgcn_alignbit(w[i], w[i], 15);
      const uint32_t x = __builtin_amdgcn_perm(hi, w[i], 0x05040100u);
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        const uint32_t s = k <= 2 ? (x << (7 - 3 * k)) : (x >> (3 * k - 7));
        const h2v v = h2_from_bits((s & 0x03800380u) | 0x3C003C00u);
        out[10 * i + 2 * k] = v[0];
        out[10 * i + 2 * k + 1] = v[1];
      }
    }
#pragma unroll
    for (int t = 10 * NW; t < NOUT; ++t) out[t] = (_Float16)1.0f;
  }
};

// ---- any other L: plain integer digits (natural order) ----
template <int L, int NW>
struct Digits<L, NW, typename std::enable_if<!(L == 3 || L == 4 || L == 5 || L == 6 || L == 8)>::type> {
  static constexpr int NV = cpw(L);
  static constexpr bool kAffine = false;
  static constexpr int kMul = 1;
  static constexpr int NOUT = ((NV * NW + 7) / 8) * 8;
  static constexpr int word_of(int t) { return t < NV * NW ? t / NV : -1; }
  static constexpr int digit_of(int t) { return t % NV; }
  __device__ static inline void run(const uint32_t (&w)[NW], _Float16 (&out)[NOUT]) {
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      uint32_t x = w[i];
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        out[NV * i + t] = (_Float16)(float)(x % (uint32_t)L);
        x /= (uint32_t)L;
      }
    }
#pragma unroll
    for (int t = NV * NW; t < NOUT; ++t) out[t] = (_Float16)0.0f;
  }
};

}  // namespace kvq
