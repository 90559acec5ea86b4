// Token ranking and tier/slot assignment (SemKV, Abstract: tokens are ranked
// by a model-internal score; the top n_hi take the higher of two adjacent
// grids; every token is kept).
//
// Rank = position in the stable descending order of the fp32 score.  It is
// computed with a least-significant-digit radix sort (4 passes of 8 bits) of
// the order-preserving u32 key, carrying the token index; each pass is
// stable, so equal scores stay in token order.  One sort segment per
// sequence.  Per pass: block histograms -> per-sequence exclusive scan ->
// stable scatter (wave ballots give each element its rank among equal
// digits of its wave, LDS counters order the waves and the rounds).
#include "common.h"
#include "internal.h"

namespace kvq {

constexpr int kSortThreads = 256;
constexpr int kSortItems = kSortTile / kSortThreads;   // 16, striped

__global__ __launch_bounds__(256) void k_key_init(const float* __restrict__ scores,
                                                  uint32_t* __restrict__ keys,
                                                  uint32_t* __restrict__ idx, int T) {
  const int b = blockIdx.y;
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T) {
    keys[(size_t)b * T + t] = score_desc_key(scores[(size_t)b * T + t]);
    idx[(size_t)b * T + t] = (uint32_t)t;
  }
}

__global__ __launch_bounds__(256) void k_hist(const uint32_t* __restrict__ keys,
                                              uint32_t* __restrict__ hist, int T, int nblk,
                                              int shift) {
  __shared__ uint32_t h[256];
  const int tid = threadIdx.x, blk = blockIdx.x, b = blockIdx.y;
  h[tid] = 0;
  __syncthreads();
  const uint32_t* kb = keys + (size_t)b * T;
  const int base = blk * kSortTile;
  for (int j = 0; j < kSortItems; ++j) {
    int i = base + j * kSortThreads + tid;
    if (i < T) atomicAdd(&h[(kb[i] >> shift) & 255u], 1u);
  }
  __syncthreads();
  hist[((size_t)b * 256 + tid) * nblk + blk] = h[tid];
}

// Exclusive scan of a 256-entry block-wide value (Hillis-Steele in LDS).
__device__ inline uint32_t block_excl_scan256(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    uint32_t t = tid >= off ? sh[tid - off] : 0u;
    __syncthreads();
    sh[tid] += t;
    __syncthreads();
  }
  uint32_t incl = sh[tid];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

// One block per sequence: exclusive scan of hist[b] laid out digit-major
// ([digit][blk]), so offsets order by digit, then by block.
__global__ __launch_bounds__(256) void k_scan(uint32_t* __restrict__ hist, int nblk) {
  __shared__ uint32_t sh[256];
  const int tid = threadIdx.x, b = blockIdx.x;
  uint32_t* hb = hist + (size_t)b * 256 * nblk;
  uint32_t sum = 0;
  for (int j = 0; j < nblk; ++j) sum += hb[tid * nblk + j];
  uint32_t total;
  uint32_t run = block_excl_scan256(sum, sh, &total);
  for (int j = 0; j < nblk; ++j) {
    uint32_t c = hb[tid * nblk + j];
    hb[tid * nblk + j] = run;
    run += c;
  }
}

__global__ __launch_bounds__(256) void k_scatter(const uint32_t* __restrict__ kin,
                                                 const uint32_t* __restrict__ iin,
                                                 uint32_t* __restrict__ kout,
                                                 uint32_t* __restrict__ iout,
                                                 const uint32_t* __restrict__ hist, int T,
                                                 int nblk, int shift) {
  __shared__ uint32_t goff[256];
  __shared__ uint32_t cnt[4][256];
  __shared__ uint32_t run[256];
  const int tid = threadIdx.x, blk = blockIdx.x, b = blockIdx.y;
  const int lane = tid & 63, w = tid >> 6;
  goff[tid] = hist[((size_t)b * 256 + tid) * nblk + blk];
  run[tid] = 0;
  const size_t sb = (size_t)b * T;
  const int base = blk * kSortTile;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < kSortItems; ++j) {
    for (int x = 0; x < 4; ++x) cnt[x][tid] = 0;
    __syncthreads();
    const int i = base + j * kSortThreads + tid;
    const bool valid = i < T;
    const uint32_t key = valid ? kin[sb + i] : 0u;
    const uint32_t d = (key >> shift) & 255u;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (d >> bit) & 1u;
      const uint64_t bb = __ballot(on);
      peers &= on ? bb : ~bb;
    }
    const uint32_t rank_w = (uint32_t)__popcll(peers & lt_mask);
    if (valid && rank_w == 0) cnt[w][d] = (uint32_t)__popcll(peers);
    __syncthreads();
    {
      const uint32_t r0 = run[tid];
      const uint32_t c0 = cnt[0][tid], c1 = cnt[1][tid], c2 = cnt[2][tid], c3 = cnt[3][tid];
      cnt[0][tid] = r0;
      cnt[1][tid] = r0 + c0;
      cnt[2][tid] = r0 + c0 + c1;
      cnt[3][tid] = r0 + c0 + c1 + c2;
      run[tid] = r0 + c0 + c1 + c2 + c3;
    }
    __syncthreads();
    if (valid) {
      const uint32_t pos = goff[d] + cnt[w][d] + rank_w;
      kout[sb + pos] = key;
      iout[sb + pos] = iin[sb + i];
    }
    __syncthreads();
  }
}

// rank[t] = sorted position; the ascending score array for the running
// median is the sorted order reversed.
__global__ __launch_bounds__(256) void k_rank_write(const uint32_t* __restrict__ idx,
                                                    const float* __restrict__ scores,
                                                    int32_t* __restrict__ ranks,
                                                    int32_t* __restrict__ ranks_out,
                                                    float* __restrict__ sorted_asc, int T,
                                                    int cap) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T) return;
  const uint32_t t = idx[(size_t)b * T + i];
  ranks[(size_t)b * T + t] = i;
  if (ranks_out) ranks_out[(size_t)b * T + t] = i;
  sorted_asc[(size_t)b * cap + (T - 1 - i)] = scores[(size_t)b * T + t];
}

__global__ __launch_bounds__(256) void k_count_hi(const int32_t* __restrict__ ranks,
                                                  uint32_t* __restrict__ bcount, int T, int nblk,
                                                  int n_hi) {
  __shared__ uint32_t sh[256];
  const int tid = threadIdx.x, blk = blockIdx.x, b = blockIdx.y;
  uint32_t c = 0;
  for (int j = 0; j < kSortItems; ++j) {
    int t = blk * kSortTile + j * kSortThreads + tid;
    if (t < T && ranks[(size_t)b * T + t] < n_hi) ++c;
  }
  uint32_t total;
  block_excl_scan256(c, sh, &total);
  if (tid == 0) bcount[(size_t)b * nblk + blk] = total;
}

// Slot = index among same-tier tokens in token order.  Each thread owns 16
// consecutive tokens; the block scans thread counts; earlier blocks' counts
// are summed directly (a sequence has at most a few dozen blocks).
__global__ __launch_bounds__(256) void k_slots(const int32_t* __restrict__ ranks,
                                               const uint32_t* __restrict__ bcount,
                                               uint32_t* __restrict__ tokmap,
                                               int32_t* __restrict__ inv_hi,
                                               int32_t* __restrict__ inv_lo,
                                               int32_t* __restrict__ counters, int T, int nblk,
                                               int n_hi, int cap, int cap_hi, int cap_lo) {
  __shared__ uint32_t sh[256];
  __shared__ uint32_t prefix;
  const int tid = threadIdx.x, blk = blockIdx.x, b = blockIdx.y;
  if (tid == 0) {
    uint32_t p = 0;
    for (int j = 0; j < blk; ++j) p += bcount[(size_t)b * nblk + j];
    prefix = p;
    if (blk == 0) {
      counters[b * 4 + 0] = T;
      counters[b * 4 + 1] = n_hi;
      counters[b * 4 + 2] = T - n_hi;
      counters[b * 4 + 3] = 0;
    }
  }
  const int t0 = blk * kSortTile + tid * kSortItems;
  bool hi[kSortItems];
  uint32_t c = 0;
  for (int j = 0; j < kSortItems; ++j) {
    int t = t0 + j;
    hi[j] = t < T && ranks[(size_t)b * T + t] < n_hi;
    c += hi[j];
  }
  uint32_t total;
  uint32_t pre = block_excl_scan256(c, sh, &total) + prefix;
  for (int j = 0; j < kSortItems; ++j) {
    int t = t0 + j;
    if (t >= T) break;
    if (hi[j]) {
      tokmap[(size_t)b * cap + t] = pre;
      inv_hi[(size_t)b * cap_hi + pre] = t;
      ++pre;
    } else {
      uint32_t slot = (uint32_t)t - pre;
      tokmap[(size_t)b * cap + t] = slot | 0x80000000u;
      inv_lo[(size_t)b * cap_lo + slot] = t;
    }
  }
}

bool launch_rank_tiers(const kvq_layout* L, uint8_t* cache, const float* scores, int T, int n_hi,
                       int32_t* ranks_out, uint8_t* ws, const QuantWs& plan, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int B = L->cfg.batch;
  const int nblk = ceil_div(T, kSortTile);
  uint32_t* keys[2] = {(uint32_t*)(ws + plan.keys[0]), (uint32_t*)(ws + plan.keys[1])};
  uint32_t* idx[2] = {(uint32_t*)(ws + plan.idx[0]), (uint32_t*)(ws + plan.idx[1])};
  uint32_t* hist = (uint32_t*)(ws + plan.hist);
  int32_t* ranks = (int32_t*)(ws + plan.ranks);
  int32_t* inv_hi = (int32_t*)(ws + plan.inv[0]);
  int32_t* inv_lo = (int32_t*)(ws + plan.inv[1]);
  uint32_t* bcount = (uint32_t*)(ws + plan.bcount);
  dim3 g256(ceil_div(T, 256), B), gblk(nblk, B);
  k_key_init<<<g256, 256, 0, s>>>(scores, keys[0], idx[0], T);
  int cur = 0;
  for (int pass = 0; pass < 4; ++pass) {
    k_hist<<<gblk, 256, 0, s>>>(keys[cur], hist, T, nblk, pass * 8);
    k_scan<<<B, 256, 0, s>>>(hist, nblk);
    k_scatter<<<gblk, 256, 0, s>>>(keys[cur], idx[cur], keys[cur ^ 1], idx[cur ^ 1], hist, T, nblk,
                                   pass * 8);
    cur ^= 1;
  }
  k_rank_write<<<g256, 256, 0, s>>>(idx[cur], scores, ranks, ranks_out,
                                    (float*)(cache + L->sorted), T, L->cfg.capacity);
  k_count_hi<<<gblk, 256, 0, s>>>(ranks, bcount, T, nblk, n_hi);
  k_slots<<<gblk, 256, 0, s>>>(ranks, bcount, (uint32_t*)(cache + L->tokmap), inv_hi, inv_lo,
                               (int32_t*)(cache + L->counters), T, nblk, n_hi, L->cfg.capacity,
                               L->cap[0], L->cap[1]);
  return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
