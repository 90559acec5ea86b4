// Internal helpers shared by the library's HIP sources (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kD = 128;          // head_dim supported by the kernels
constexpr int kGqa = 4;          // query heads per KV head
constexpr int kTile = 16;        // slots per key tile

// Bits of counters[b][3]: the pool of the new token was full (append), and a
// value group scale of 1024 or more is stored (the decode kernels then scale
// their fp16 value operand down).
constexpr int kFlagPoolFull = 1;
constexpr int kFlagBigValueScale = 2;
constexpr uint32_t kBigScaleBits = 0x6400u;   // fp16 1024.0

// Cache policy of loads whose data a kernel reads exactly once (the decode's
// packed words and (scale, zero) pairs, the fp16 rows quantize reads):
// non-temporal (the `nt` bit), a hint that the data is streamed.  Measured
// on MI355X: a 16-byte read stream runs at 6.9 instead of 6.1 TB/s with it,
// the decode pools 2-4 % faster at unchanged counted HBM traffic.  It pays
// only where each load instruction covers whole 128-byte lines: quantize's
// row gather read 64-byte halves with four lanes per row, and with the
// policy it fetched 5.6 % more and ran 3-7 % slower; with eight lanes per
// row it reads whole lines.
constexpr int kStreamPolicy = 2;

// 16 bytes (16-byte aligned) of a read-once stream, non-temporal.
__device__ inline uint4 ld_stream16(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Sets kFlagBigValueScale of sequence b when any lane of the wave formed a
// value scale (fp16 bits s_bits, non-negative) of 1024 or more: one atomic
// per wave, only in waves that hold one.
__device__ inline void flag_big_value_scale(int32_t* counters, int b, uint32_t s_bits) {
  const unsigned long long m = __ballot((s_bits & 0x7FFFu) >= kBigScaleBits);
  if (__builtin_expect(m != 0ull, 0) && (int)(threadIdx.x & 63) == __builtin_ctzll(m))
    atomicOr(counters + b * 4 + 3, kFlagBigValueScale);
}

// Base-L digits per 32-bit word: max{n : L^n <= 2^32}.
__host__ __device__ inline int codes_per_word(int L) {
  uint64_t p = 1;
  int n = 0;
  while (p * (uint64_t)L <= (1ull << 32)) {
    p *= (uint64_t)L;
    ++n;
  }
  return n;
}

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// fp16 bits -> integer key in IEEE total order (-0 below +0).
__device__ inline int f16_order_key(uint32_t b) {
  return (b & 0x8000u) ? -(int)(b & 0x7FFFu) - 1 : (int)b;
}
__device__ inline uint32_t f16_from_order_key(int k) {
  return k < 0 ? (uint32_t)((-(k + 1)) | 0x8000) : (uint32_t)k;
}

__device__ inline float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)bits16));
}
__device__ inline uint32_t f2h_rne(float x) {
  return (uint32_t)__half_as_ushort(__float2half_rn(x));
}

// Quantize one group given its fp16 min/max (bits).  Produces the fp16 scale
// bits and the fp32 values the per-value step needs.  The per-value code is
//   c = clamp(rint(fl32(x - z) / s), 0, L-1)
// where the quotient is computed as q0 = a*r, rho = fma(-q0, s, a),
// q = fma(rho, r, q0) with r = RN(1/s): Markstein's correction, which returns
// the correctly rounded fp32 quotient when r is the correctly rounded
// reciprocal (no overflow/underflow for fp16-range operands).
struct GroupQ {
  float z, s, r;
  uint32_t s_bits;
  float top;
};

// RN(a / d) for a = 0 or a in [2^-24, 2^17] (every difference of two fp16
// values) and d in 2..7, without the IEEE division sequence: the quotient
// correction q = fma(fma(-q0, d, a), r, q0), q0 = a * r, r = RN(1/d)
// (Markstein) returns the correctly rounded quotient for d = 2, 3, 4, 5, 7
// on that whole domain (checked exhaustively against IEEE division); for
// d = 6 it does not, so a is halved first (exact there) and divided by 3.
__device__ inline float div_by_small(float a, int d) {
  if (d < 2 || d > 7) return a / (float)d;        // outside the checked set: IEEE division
  if (d == 6) {
    a *= 0.5f;
    d = 3;
  }
  const float df = (float)d;
  const float r = 1.0f / df;                      // folded at compile time for constant d
  const float q0 = a * r;
  const float rho = __builtin_fmaf(-q0, df, a);
  return __builtin_fmaf(rho, r, q0);
}

// RN(1 / s) for a positive finite fp16 value s: the hardware reciprocal and
// one Newton step (checked on the device against IEEE division for every
// such s).
__device__ inline float recip_f16_exact(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(r0, e, r0);
}

__device__ inline GroupQ group_setup(uint32_t mn_bits, uint32_t mx_bits, int L) {
  GroupQ g;
  g.z = h2f(mn_bits);
  const float range = h2f(mx_bits) - g.z;         // fp32, round to nearest even
  float s32 = div_by_small(range, L - 1);         // = RN(range / (L-1))
  // keep the fp32 rounding: without this the compiler may fuse the last fma
  // with the fp16 conversion (one rounding instead of fp32 then fp16)
  asm volatile("" : "+v"(s32));
  g.s_bits = f2h_rne(s32);
  g.s = h2f(g.s_bits);
  g.r = (g.s != 0.0f) ? recip_f16_exact(g.s) : 0.0f;   // = RN(1 / s)
  g.top = (float)(L - 1);
  return g;
}

__device__ inline uint32_t quant_value(float x, const GroupQ& g) {
  if (g.s == 0.0f) return 0u;
  float a = x - g.z;
  float q0 = a * g.r;
  float rho = __builtin_fmaf(-q0, g.s, a);
  float q = __builtin_fmaf(rho, g.r, q0);
  float c = __builtin_rintf(q);
  c = fminf(fmaxf(c, 0.0f), g.top);
  return (uint32_t)c;
}

// Order-preserving u32 key of an fp32 score for a DESCENDING sort expressed
// as an ascending one; -0 is folded onto +0 so equal scores tie.
__device__ inline uint32_t score_desc_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

}  // namespace kvq
