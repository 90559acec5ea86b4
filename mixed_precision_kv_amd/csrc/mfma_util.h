// Small helpers shared by the matrix-core decode kernels: the partial
// record, DPP row reductions, the head reduce-scatter and raw buffer loads
// (out-of-range offsets read 0).
#pragma once
#include <stdint.h>

#include "common.h"

namespace kvq {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kPartF = 4 + kD;      // floats per head in a partial: m, l, pad, pad, acc[128]
constexpr float kAScale = 64.0f;    // value-operand weights carry 2^6 (fp16 range)
constexpr float kBigValueShift = 64.0f;   // flagged sequences: value scales enter as s / 2^6

// fp16 value scale of a (scale, zero) word as the factor of the value
// operand A = 2^6 p * s.  p <= 1, so A <= 2^6 s, which is finite for
// s < 1024; a sequence holding a larger value scale is flagged by the
// quantizers and its scales enter divided by 2^6 (exact unless subnormal).
__device__ inline _Float16 value_scale_operand(uint32_t meta, bool big) {
  const uint16_t sb = (uint16_t)(meta & 0xFFFFu);
  return big ? (_Float16)(h2f(sb) * (1.0f / kBigValueShift)) : __builtin_bit_cast(_Float16, sb);
}

__device__ inline float dpp_ror(float v, int n) {
  // row_ror:n within each row of 16 lanes
  int x = __float_as_int(v);
  int r;
  switch (n) {
    case 8: r = __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(x, x, 0x122, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(x, x, 0x121, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}
__device__ inline float row_max16(float v) {
  v = fmaxf(v, dpp_ror(v, 8));
  v = fmaxf(v, dpp_ror(v, 4));
  v = fmaxf(v, dpp_ror(v, 2));
  v = fmaxf(v, dpp_ror(v, 1));
  return v;
}
__device__ inline float row_sum16(float v) {
  v += dpp_ror(v, 8);
  v += dpp_ror(v, 4);
  v += dpp_ror(v, 2);
  v += dpp_ror(v, 1);
  return v;
}

// Lane (n, g) holds x[h], h = 0..3, for slot n and sub-group g.  Returns, in
// lane (n, r), the sum over g of x[r] (r = lane / 16).
__device__ inline float reduce_scatter4(f4 x) {
  auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[2]), false, false);
  auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]), __float_as_uint(x[3]), false, false);
  const float y0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float y1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(y0), __float_as_uint(y1), false, false);
  return __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
}

// Orders one wave's LDS accesses: its stores land before the loads that
// follow (the wave's own LDS operations complete in issue order).
__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __amdgpu_buffer_rsrc_t BufRes;
constexpr uint32_t kOutOfRange = 0x80000000u;   // beyond every region: reads 0

__device__ inline BufRes make_res(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline uint32_t bload(BufRes r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kStreamPolicy);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ inline u32x2 bload2(BufRes r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)byte_off, 0, kStreamPolicy);
}

}  // namespace kvq
