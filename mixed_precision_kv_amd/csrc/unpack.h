// Base-L digits of packed words as fp16 matrix operands (decode kernel).
//
// L in {3, 5, 6, 7}: a word is cut into chunks of four base-L digits by exact
// integer division by B = L^4, and each chunk (x < B) indexes a table in LDS
// whose entry holds its four digits as fp16: four consecutive elements of a
// matrix operand, fetched by one 8-byte LDS read.  Division by the constant B
// is a multiply-high by a rounded-up reciprocal and a shift (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with M = ceil(2^(32+s) / B) and e = M B - 2^(32+s), floor(x M / 2^(32+s))
// equals floor(x / B) whenever e (X - 1) < 2^(32+s) for all x < X; the
// constants are searched at compile time per level with X the range of the
// value divided there.  The chunks of a lane's words fill its operand in
// order: digit d of chunk k of word i is element 4 (i NC + k) + d.  The top
// chunk of a word may hold fewer than four digits; its missing digits are 0.
//
// L in {4, 8}: bit fields injected into fp16 mantissas (Digits<4/8>); these
// give the affine value 1 + d/M, which the kernel folds into (scale, zero).
#pragma once
#include <stdint.h>

#include <type_traits>

#include "digits.h"

namespace kvq {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

struct DivMagic {
  uint32_t M;
  int S;
};

// floor(x / B) == mulhi(x, M) >> S for every x < X (S = -1: none found).
__host__ __device__ constexpr DivMagic div_magic(uint32_t B, uint64_t X) {
  for (int s = 0; s < 32; ++s) {
    const uint64_t p2 = 1ull << (32 + s);
    const uint64_t M = (p2 + B - 1) / B;
    if (M >= (1ull << 32)) continue;
    const uint64_t e = M * B - p2;
    if (e * (X - 1) < p2) return DivMagic{(uint32_t)M, s};
  }
  return DivMagic{0, -1};
}

template <int L>
struct ChunkTable {
  static constexpr int NV = cpw(L);                 // digits per word
  static constexpr int NC = (NV + 3) / 4;           // chunks per word
  static constexpr uint32_t B = ipow(L, 4);         // table entries
  // exclusive bound of the value divided at level k (level 0: the word)
  static constexpr uint64_t range(int k) {
    uint64_t X = 1;
    for (int i = 0; i < NV; ++i) X *= (uint64_t)L;
    for (int i = 0; i < k; ++i) X = (X + B - 1) / B;
    return X;
  }
  struct Mags {
    DivMagic m[NC - 1];
  };
  static constexpr Mags make_mags() {
    Mags r{};
    for (int k = 0; k < NC - 1; ++k) r.m[k] = div_magic(B, range(k));
    return r;
  }
  static constexpr Mags kMag = make_mags();
  static constexpr bool mags_ok() {
    for (int k = 0; k < NC - 1; ++k)
      if (kMag.m[k].S < 0) return false;
    return range(NC - 1) <= B;
  }
  static_assert(mags_ok(), "no exact reciprocal for this grid");

  // Byte offsets (8 x chunk) of the NC chunks of word w, least significant
  // first.  The top chunk is clamped to the table so that a corrupted word
  // cannot index past it.
  __device__ static inline void offsets(uint32_t w, uint32_t* off) {
    uint32_t x = w;
#pragma unroll
    for (int k = 0; k < NC - 1; ++k) {
      const uint32_t q = __umulhi(x, kMag.m[k].M) >> kMag.m[k].S;
      off[k] = (x - q * B) * 8u;
      x = q;
    }
    off[NC - 1] = min(x, B - 1u) * 8u;
  }

  // Entry x: digits 0..3 of x as fp16 (digit d in half d).
  __device__ static inline void fill(uint2* tab, int tid, int nthr) {
    for (int x = tid; x < (int)B; x += nthr) {
      uint32_t v = (uint32_t)x;
      uint32_t h[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        h[d] = __builtin_bit_cast(uint16_t, (_Float16)(float)(v % (uint32_t)L));
        v /= (uint32_t)L;
      }
      tab[x] = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
};

template <int L, int NW>
struct TableUnpack {
  using CT = ChunkTable<L>;
  static constexpr int NV = CT::NV, NC = CT::NC, PW = 4 * NC;
  static constexpr bool kTable = true, kAffine = false;
  static constexpr int kMul = 1;
  static constexpr int kTableEntries = (int)CT::B;
  static constexpr int NCH = NW * NC;                  // chunks per call
  static constexpr int NH8 = (NCH + 1) / 2;            // operands per call
  static constexpr int NOUT = 8 * NH8;
  static constexpr int word_of(int t) { return (t < NW * PW && t % PW < NV) ? t / PW : -1; }
  static constexpr int digit_of(int t) { return t % PW; }
  static constexpr int pos_of(int word, int digit) { return word * PW + digit; }
  __device__ static inline void fill(uint2* tab, int tid, int nthr) { CT::fill(tab, tid, nthr); }
  __device__ static inline void run(const uint32_t (&w)[NW], const uint2* tab, h8 (&out)[NH8]) {
    uint32_t off[2 * NH8];
#pragma unroll
    for (int i = 0; i < NW; ++i) CT::offsets(w[i], off + i * NC);
    const char* base = reinterpret_cast<const char*>(tab);
#pragma unroll
    for (int m = 0; m < NH8; ++m) {
      const uint2 a = *reinterpret_cast<const uint2*>(base + off[2 * m]);
      const uint2 b = (2 * m + 1 < NCH) ? *reinterpret_cast<const uint2*>(base + off[2 * m + 1])
                                        : make_uint2(0u, 0u);
      const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
      out[m] = __builtin_bit_cast(h8, v);
    }
  }
};

template <int L, int NW>
struct BitUnpack {
  using D = Digits<L, NW>;
  static constexpr int NV = D::NV;
  static constexpr bool kTable = false, kAffine = D::kAffine;
  static constexpr int kMul = D::kMul;
  static constexpr int kTableEntries = 1;
  static constexpr int NOUT = D::NOUT;
  static constexpr int NH8 = NOUT / 8;
  static constexpr int word_of(int t) { return D::word_of(t); }
  static constexpr int digit_of(int t) { return D::digit_of(t); }
  // inverse of (word_of, digit_of): digits k and k + NV/2 of a word share a
  // register, words are blocks of NV outputs
  static constexpr int pos_of(int word, int digit) {
    return word * NV + (digit < NV / 2 ? 2 * digit : 2 * (digit - NV / 2) + 1);
  }
  static constexpr bool pos_ok() {
    for (int t = 0; t < NV * NW; ++t)
      if (pos_of(D::word_of(t), D::digit_of(t)) != t) return false;
    return true;
  }
  static_assert(pos_ok(), "operand position map");
  __device__ static inline void fill(uint2*, int, int) {}
  __device__ static inline void run(const uint32_t (&w)[NW], const uint2*, h8 (&out)[NH8]) {
    _Float16 dg[NOUT];
    D::run(w, dg);
#pragma unroll
    for (int m = 0; m < NH8; ++m)
#pragma unroll
      for (int i = 0; i < 8; ++i) out[m][i] = dg[8 * m + i];
  }
};

template <int L, int NW>
using Unpack = typename std::conditional<(L == 4 || L == 8), BitUnpack<L, NW>, TableUnpack<L, NW>>::type;

}  // namespace kvq
