// Base-L digits of packed words as fp16 matrix operands: the power-of-two
// grids (L = 4, 8), plus small fp16 helpers shared with the quantize kernels.
//
// Power-of-two grids need no arithmetic: a digit field is or-ed into the
// mantissa of fp16 1.0, giving the affine value 1 + d/M (M = 4 or 8); the
// decode kernel folds the affine map into the group's (scale, zero).
#pragma once
#include <stdint.h>

#include "tiling.h"

namespace kvq {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

__device__ inline h2v h2_from_bits(uint32_t b) { return __builtin_bit_cast(h2v, b); }

// (x & m) | c in one instruction (three-input bitwise op, truth table 0xEA
// for inputs with patterns 0xF0, 0xCC, 0xAA)
__device__ inline uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(x, m, c, 0xEA);
}

__host__ __device__ constexpr uint32_t ipow(uint32_t L, int k) {
  uint32_t p = 1;
  for (int i = 0; i < k; ++i) p *= L;
  return p;
}

// Extraction of NW words of L levels into fp16 values.  Output element t
// holds digit digit_of(t) of word word_of(t) (or is padding, word_of < 0).
template <int L, int NW>
struct Digits;

// ---- L = 4: 2-bit fields, digits (k, k+8) share a register ----
template <int NW>
struct Digits<4, NW> {
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
        const h2v v = h2_from_bits(and_or(s, 0x03000300u, 0x3C003C00u));
        out[16 * i + 2 * k] = v[0];
        out[16 * i + 2 * k + 1] = v[1];
      }
  }
};

// ---- L = 8: 3-bit fields; the high 16 digits' bits are realigned so digits
// (k, k+5) share a register ----
template <int NW>
struct Digits<8, NW> {
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
        const h2v v = h2_from_bits(and_or(s, 0x03800380u, 0x3C003C00u));
        out[10 * i + 2 * k] = v[0];
        out[10 * i + 2 * k + 1] = v[1];
      }
    }
#pragma unroll
    for (int t = 10 * NW; t < NOUT; ++t) out[t] = (_Float16)1.0f;
  }
};

}  // namespace kvq
