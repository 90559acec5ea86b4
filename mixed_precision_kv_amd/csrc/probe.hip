// Read-stream probe: the achievable HBM read bandwidth of this device, the
// second reference (beside the published 8 TB/s) against which the decode
// and quantize rates are reported.  Every byte of the buffer is read once
// with 16-byte non-temporal loads (the policy the kernels use for their
// read-once streams), each workgroup a contiguous slab, coalesced per wave;
// the xor of everything read is kept so the loads cannot be dropped.
#include "common.h"
#include "internal.h"

namespace kvq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256, kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4* __restrict__ src, size_t n16,
                                                               uint32_t* __restrict__ sink) {
  // workgroup g reads the contiguous slab [g * slab, (g + 1) * slab) of
  // 16-byte vectors, kProbeUnroll x 4 KB per trip
  const size_t slab = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t s0 = (size_t)blockIdx.x * slab, s1 = s0 + slab < n16 ? s0 + slab : n16;
  uint32_t acc = 0;
  for (size_t i0 = s0 + threadIdx.x; i0 < s1; i0 += (size_t)kProbeThreads * kProbeUnroll) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) {
      const size_t i = i0 + (size_t)k * kProbeThreads;
      v[k] = i < s1 ? __builtin_nontemporal_load(src + i) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  // one word per workgroup: the xor of its threads
  __shared__ uint32_t red[kProbeThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int t = 0; t < kProbeThreads; ++t) x ^= red[t];
    sink[blockIdx.x] = x;
  }
}

bool launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int nwg, void* stream) {
  k_stream_read<<<nwg, kProbeThreads, 0, (hipStream_t)stream>>>((const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
