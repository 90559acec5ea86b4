// Token ranking and tier/slot assignment (SemKV, Abstract: tokens are ranked
// by a model-internal score; the top n_hi take the higher of two adjacent
// grids; every token is kept).
//
// Rank = position in the stable descending order of the fp32 score, i.e. the
// ascending order of an order-preserving u32 key with ties in token order.
// Each block of kBlkSort tokens is sorted in LDS (4 stable passes of 8
// bits); each sorted element's rank is then its position in its own block
// plus, for every other block, the number of that block's keys that precede
// it: keys that are smaller, and equal keys of earlier blocks (branch-free
// binary searches over sorted keys held in LDS).  Up to kMergeMaxT tokens all
// of a sequence's sorted keys fit one workgroup's LDS; longer sequences take
// the other blocks kMergeBlocks at a time and add partial counts.  Slots
// (index among same-tier tokens in token order) come from one scan per
// sequence.
#include "common.h"
#include "internal.h"

namespace kvq {

// Workgroups are handed to the 8 XCDs round-robin by linear id, and each XCD
// has its own L2.  The sort kernels run on a 1-D grid of X * ceil(B / X) *
// nblk workgroups, X = min(B, 8), mapped so that every block of sequence b
// runs on the XCDs congruent to b mod X: with 8 or more sequences each one's
// scattered 4-byte writes meet in one L2, and fewer sequences still spread
// over every XCD.
constexpr int kXcds = 8;
__host__ __device__ inline int seq_group(int B) { return B < kXcds ? B : kXcds; }
__device__ inline bool seq_block(int nblk, int B, int& b, int& blk) {
  const int X = seq_group(B);
  const int id = blockIdx.x, x = id % X, k = id / X;
  b = x + X * (k / nblk);
  blk = k % nblk;
  return b < B;
}
static inline dim3 seq_grid(int nblk, int B) {
  const int X = seq_group(B);
  return dim3(X * ((B + X - 1) / X) * nblk);
}

// Slot = index among same-tier tokens in token order.  Workgroup (seg, b)
// owns tokens [seg * SEG, (seg + 1) * SEG); earlier segments' high-tier
// counts give its base; wave w owns a contiguous quarter, read in
// 64-token chunks (coalesced) with ballots for the in-chunk prefix.
template <int SEG>
__global__ __launch_bounds__(256) void k_rank_slots(const int32_t* __restrict__ ranks,
                                                    const uint32_t* __restrict__ segcnt,
                                                    uint32_t* __restrict__ tokmap,
                                                    int32_t* __restrict__ inv_hi,
                                                    int32_t* __restrict__ inv_lo,
                                                    int32_t* __restrict__ pos_hi,
                                                    int32_t* __restrict__ pos_lo,
                                                    int32_t* __restrict__ counters, int T, int n_hi,
                                                    int cap, int cap_hi, int cap_lo, int nseg, int B) {
  constexpr int kChunks = SEG / 4 / 64;               // 64-token chunks per wave
  __shared__ uint32_t wtot[4];
  __shared__ uint32_t wbase[4];
  const int tid = threadIdx.x;
  int b, seg;
  if (!seq_block(nseg, B, b, seg)) return;
  const int lane = tid & 63, w = tid >> 6;
  {
    // high-tier tokens of the earlier segments, summed by every thread
    uint32_t p = 0;
    for (int k = tid; k < seg; k += 256) p += segcnt[(size_t)b * nseg + k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) p += (uint32_t)__shfl_xor((int)p, o);
    if (lane == 0) wbase[w] = p;
  }
  if (tid == 0) {
    if (seg == 0) {
      counters[b * 4 + 0] = T;
      counters[b * 4 + 1] = n_hi;
      counters[b * 4 + 2] = T - n_hi;
      counters[b * 4 + 3] = 0;
    }
  }
  const int t0 = seg * SEG + w * (SEG / 4);
  const int32_t* rb = ranks + (size_t)b * T;
  uint64_t m[kChunks];
  uint32_t mine = 0;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int t = t0 + k * 64 + lane;
    m[k] = __ballot(t < T && rb[t] < n_hi);
    mine += (uint32_t)__popcll(m[k]);
  }
  if (lane == 0) wtot[w] = mine;
  __syncthreads();
  uint32_t pre = wbase[0] + wbase[1] + wbase[2] + wbase[3];
  for (int k = 0; k < w; ++k) pre += wtot[k];
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int t = t0 + k * 64 + lane;
    if (t < T) {
      const uint32_t hb = pre + (uint32_t)__popcll(m[k] & lt_mask);   // high-tier tokens before t
      if ((m[k] >> lane) & 1ull) {
        tokmap[(size_t)b * cap + t] = hb;
        inv_hi[(size_t)b * cap_hi + hb] = t;
        if (pos_hi) pos_hi[(size_t)b * cap_hi + hb] = t;   // pre-RoPE keys: slot -> position
      } else {
        const uint32_t slot = (uint32_t)t - hb;
        tokmap[(size_t)b * cap + t] = slot | 0x80000000u;
        inv_lo[(size_t)b * cap_lo + slot] = t;
        if (pos_lo) pos_lo[(size_t)b * cap_lo + slot] = t;
      }
    }
    pre += (uint32_t)__popcll(m[k]);
  }
}

// ---------------- sequences of up to kMergeMaxT tokens ----------------

constexpr int kBlkSort = 4096;               // keys per block of the block sort
constexpr int kBlkThreads = 1024;            // 16 waves x 4 chunks of 64

// Stable sort of one block of kBlkSort keys in LDS, 4 passes of 8 bits.
// Wave w owns elements [256 w, 256 w + 256) in 64-element chunks, in order;
// an element goes to (keys with a smaller digit) + (same digit in earlier
// waves) + (same digit earlier in its own wave, from the wave's running
// counts).  Out of range elements carry the largest key and the largest
// indices, so they sort last.  Also clears the block's high-tier counts and,
// for long sequences, the partial counts of its elements.
__global__ __launch_bounds__(kBlkThreads) void k_rank_block_sort(const float* __restrict__ scores,
                                                                 uint32_t* __restrict__ skeys,
                                                                 uint32_t* __restrict__ sidx,
                                                                 uint32_t* __restrict__ hicnt,
                                                                 uint32_t* __restrict__ cnt, int T,
                                                                 int ld, int nblk, int B) {
  constexpr int NW = kBlkThreads / 64;
  __shared__ uint32_t kb[kBlkSort];
  __shared__ uint16_t ib[kBlkSort];
  __shared__ uint32_t wrun[NW][256];         // per wave: running count of each digit
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int b, blk;
  if (!seq_block(nblk, B, b, blk)) return;
  {
    const int nseg = (T + kSortTile - 1) / kSortTile, seg = blk * (kBlkSort / kSortTile) + tid;
    if (tid < kBlkSort / kSortTile && seg < nseg) hicnt[(size_t)b * nseg + seg] = 0u;
  }
  const int base = blk * kBlkSort, nb = min(kBlkSort, T - base);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t key[4], ix[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = 256 * w + 64 * c + lane;
    key[c] = e < nb ? score_desc_key(scores[(size_t)b * T + base + e]) : 0xFFFFFFFFu;
    ix[c] = (uint32_t)e;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    for (int i = tid; i < NW * 256; i += kBlkThreads) (&wrun[0][0])[i] = 0u;
    __syncthreads();
    uint32_t d[4], pin[4];                   // digit; rank among equal digits of the wave
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      d[c] = (key[c] >> shift) & 255u;
      uint64_t peers = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const bool on = (d[c] >> bit) & 1u;
        const uint64_t bb = __ballot(on);
        peers &= on ? bb : ~bb;
      }
      const uint64_t below = peers & lt_mask;
      const uint32_t before = wrun[w][d[c]];   // this digit in earlier chunks of the wave
      pin[c] = before + (uint32_t)__popcll(below);
      if (below == 0ull) wrun[w][d[c]] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();
    // threads 0..255 (digit tid): exclusive scan of the totals, per-wave bases
    uint32_t tw[NW], tot = 0, inc = 0;
    if (tid < 256) {
#pragma unroll
      for (int x = 0; x < NW; ++x) { tw[x] = wrun[x][tid]; tot += tw[x]; }
      inc = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)inc, o);
        if (lane >= o) inc += y;
      }
      if (lane == 63) wsum[w] = inc;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t run = inc - tot;
      for (int x = 0; x < w; ++x) run += wsum[x];
#pragma unroll
      for (int x = 0; x < NW; ++x) { wrun[x][tid] = run; run += tw[x]; }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t pos = wrun[w][d[c]] + pin[c];
      kb[pos] = key[c];
      ib[pos] = (uint16_t)ix[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 256 * w + 64 * c + lane;
      key[c] = kb[e];
      ix[c] = ib[e];
    }
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = 256 * w + 64 * c + lane;
    if (e < nb) {
      skeys[(size_t)b * ld + base + e] = key[c];
      sidx[(size_t)b * ld + base + e] = (uint32_t)base + ix[c];
      if (cnt) cnt[(size_t)b * ld + base + e] = 0u;
    }
  }
}

struct MergeArgs {
  const uint32_t* skeys;        // sorted keys per block, [b][ld] (ld: T rounded up to 4)
  const uint32_t* sidx;         // their token indices
  const float* scores;
  int32_t* ranks;
  int32_t* ranks_out;
  float* sorted_asc;
  uint32_t* hicnt;              // high-tier tokens per kSortTile tokens, [b][ceil(T / kSortTile)]
  uint32_t* cnt;                // long sequences: entries of other blocks before each element, [b][ld]
  int T, ld, nblk, n_hi, cap, B;
  int ngrp;                     // long sequences: groups of kMergeBlocks blocks
};

// LDS word of sorted key i: one pad word per 32 and per 1024 keys, so that
// the probes of one binary-search step (indices that differ by multiples of
// the step) fall in different banks.
__device__ inline int sk_slot(int i) { return i + (i >> 5) + (i >> 10); }
constexpr int kSkWords = kMergeMaxT + kMergeMaxT / 32 + kMergeMaxT / 1024;

// Entries of the sorted block at `first` that precede key x: entries < xe
// with xe = x + 1 when the block holds earlier tokens (equal keys count),
// else xe = x.  Entries past the block's end hold the largest key, which
// never counts.  Fixed trip count, no branches.
__device__ inline int count_before(const uint32_t* sk, int first, uint32_t xe) {
  const uint32_t* blk = sk + sk_slot(first);          // first: a multiple of 1024
  int pos = 0;
#pragma unroll
  for (int step = kBlkSort / 2; step > 0; step >>= 1) {
    const uint32_t y = blk[sk_slot(pos + step - 1)];
    pos += y < xe ? step : 0;
  }
  return pos + (blk[sk_slot(pos)] < xe ? 1 : 0);
}

// Rank r of sorted element p of block blk (when valid): ranks, the ascending
// score array, and the high-tier counts per kSortTile-token range.
__device__ inline void write_rank(const MergeArgs& a, int b, int blk, int p, bool valid, int r,
                                  uint32_t* whi) {
  const int tid = threadIdx.x, base = blk * kBlkSort;
  if (tid < kBlkSort / kSortTile) whi[tid] = 0u;
  __syncthreads();
  if (valid) {
    const uint32_t tok = a.sidx[(size_t)b * a.ld + base + p];
    a.ranks[(size_t)b * a.T + tok] = r;
    if (a.ranks_out) a.ranks_out[(size_t)b * a.T + tok] = r;
    a.sorted_asc[(size_t)b * a.cap + (a.T - 1 - r)] = a.scores[(size_t)b * a.T + tok];
    if (r < a.n_hi) atomicAdd(&whi[(tok - base) / kSortTile], 1u);
  }
  __syncthreads();
  const int nseg = (a.T + kSortTile - 1) / kSortTile, seg = base / kSortTile + tid;
  if (tid < kBlkSort / kSortTile && seg < nseg && whi[tid])
    atomicAdd(&a.hicnt[(size_t)b * nseg + seg], whi[tid]);
}

// Rank of 1024 sorted elements of one block (quarter q): the element's
// position in its block plus the entries of every other block that precede
// it.  One thread per element; the sequence's sorted keys sit in LDS.
__global__ __launch_bounds__(1024) void k_rank_merge(MergeArgs a) {
  __shared__ uint32_t sk[kSkWords];
  __shared__ uint32_t whi[kBlkSort / kSortTile];
  const int tid = threadIdx.x;
  int b, bq;
  if (!seq_block(a.nblk * 4, a.B, b, bq)) return;
  const int blk = bq >> 2, p = (bq & 3) * 1024 + tid;   // sorted position in the block
  {
    // the sequence's sorted keys into LDS: 16-byte loads, all in flight
    const uint32_t* src = a.skeys + (size_t)b * a.ld;
    const int n4 = a.T >> 2;
    const uint4* src4 = reinterpret_cast<const uint4*>(src);
    uint4 v[kMergeMaxT / 4 / 1024];
#pragma unroll
    for (int k = 0; k < kMergeMaxT / 4 / 1024; ++k) {
      const int i = tid + 1024 * k;
      if (i < n4) v[k] = src4[i];
    }
#pragma unroll
    for (int k = 0; k < kMergeMaxT / 4 / 1024; ++k) {
      const int i = tid + 1024 * k;
      if (i < n4) {
        const int o = sk_slot(4 * i);        // 4 i .. 4 i + 3 share their pad count
        sk[o] = v[k].x; sk[o + 1] = v[k].y; sk[o + 2] = v[k].z; sk[o + 3] = v[k].w;
      }
    }
    if (tid < (a.T & 3)) sk[sk_slot(4 * n4 + tid)] = src[4 * n4 + tid];
    for (int i = a.T + tid; i < a.nblk * kBlkSort; i += 1024) sk[sk_slot(i)] = 0xFFFFFFFFu;
  }
  __syncthreads();
  const int base = blk * kBlkSort, nb = min(kBlkSort, a.T - base);
  const bool valid = p < nb;
  const uint32_t x = sk[sk_slot(base + (valid ? p : 0))];
  int r = p;
  constexpr int NI = kMergeMaxT / kBlkSort;            // blocks of the longest sequence
  int c[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bool use = i < a.nblk && i != blk;
    const int n = use ? min(kBlkSort, a.T - i * kBlkSort) : 0;
    // equal keys of earlier blocks count; x = 0xFFFFFFFF: every entry does
    if (i < blk && x == 0xFFFFFFFFu) c[i] = use ? n : 0;
    else c[i] = use ? count_before(sk, i * kBlkSort, i < blk ? x + 1u : x) : 0;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) r += c[i];
  write_rank(a, b, blk, p, valid, r, whi);
}

// Groups of kMergeBlocks sorted blocks (kMergeMaxT keys) fit one workgroup's
// LDS; longer sequences count, per (element quarter, group), the entries of
// the group's blocks that precede each element and add them to its partial
// count; k_rank_finish then writes the ranks.
constexpr int kMergeBlocks = kMergeMaxT / kBlkSort;
__global__ __launch_bounds__(1024) void k_rank_merge_part(MergeArgs a) {
  __shared__ uint32_t sk[kSkWords];
  const int tid = threadIdx.x;
  int b, bg;
  if (!seq_block(a.nblk * 4 * a.ngrp, a.B, b, bg)) return;
  const int bq = bg % (a.nblk * 4), gi = bg / (a.nblk * 4);
  const int blk = bq >> 2, p = (bq & 3) * 1024 + tid;
  const int g0 = gi * kMergeMaxT, gn = min(kMergeMaxT, a.T - g0);
  {
    const uint32_t* src = a.skeys + (size_t)b * a.ld + g0;
    const int n4 = gn >> 2;
    const uint4* src4 = reinterpret_cast<const uint4*>(src);
    uint4 v[kMergeMaxT / 4 / 1024];
#pragma unroll
    for (int k = 0; k < kMergeMaxT / 4 / 1024; ++k) {
      const int i = tid + 1024 * k;
      if (i < n4) v[k] = src4[i];
    }
#pragma unroll
    for (int k = 0; k < kMergeMaxT / 4 / 1024; ++k) {
      const int i = tid + 1024 * k;
      if (i < n4) {
        const int o = sk_slot(4 * i);
        sk[o] = v[k].x; sk[o + 1] = v[k].y; sk[o + 2] = v[k].z; sk[o + 3] = v[k].w;
      }
    }
    if (tid < (gn & 3)) sk[sk_slot(4 * n4 + tid)] = src[4 * n4 + tid];
    for (int i = gn + tid; i < kMergeMaxT; i += 1024) sk[sk_slot(i)] = 0xFFFFFFFFu;
  }
  __syncthreads();
  const int base = blk * kBlkSort, nb = min(kBlkSort, a.T - base);
  if (p >= nb) return;
  const uint32_t x = a.skeys[(size_t)b * a.ld + base + p];
  int r = 0;
  int c[kMergeBlocks];
#pragma unroll
  for (int i = 0; i < kMergeBlocks; ++i) {
    const int gb = gi * kMergeBlocks + i;
    const bool use = gb < a.nblk && gb != blk;
    const int n = use ? min(kBlkSort, a.T - gb * kBlkSort) : 0;
    if (gb < blk && x == 0xFFFFFFFFu) c[i] = use ? n : 0;
    else c[i] = use ? count_before(sk, i * kBlkSort, gb < blk ? x + 1u : x) : 0;
  }
#pragma unroll
  for (int i = 0; i < kMergeBlocks; ++i) r += c[i];
  if (r) atomicAdd(&a.cnt[(size_t)b * a.ld + base + p], (uint32_t)r);
}

__global__ __launch_bounds__(1024) void k_rank_finish(MergeArgs a) {
  __shared__ uint32_t whi[kBlkSort / kSortTile];
  const int tid = threadIdx.x;
  int b, bq;
  if (!seq_block(a.nblk * 4, a.B, b, bq)) return;
  const int blk = bq >> 2, p = (bq & 3) * 1024 + tid;
  const int base = blk * kBlkSort, nb = min(kBlkSort, a.T - base);
  const bool valid = p < nb;
  const int r = valid ? p + (int)a.cnt[(size_t)b * a.ld + base + p] : 0;
  write_rank(a, b, blk, p, valid, r, whi);
}

bool launch_rank_tiers(const kvq_layout* L, uint8_t* cache, const float* scores, int T, int n_hi,
                       int32_t* ranks_out, uint8_t* ws, const QuantWs& plan, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int B = L->cfg.batch;
  const int nblk = ceil_div(T, kSortTile);
  uint32_t* keys[2] = {(uint32_t*)(ws + plan.keys[0]), (uint32_t*)(ws + plan.keys[1])};
  uint32_t* sidx = (uint32_t*)(ws + plan.idx);
  uint32_t* segcnt = (uint32_t*)(ws + plan.segcnt);
  int32_t* ranks = (int32_t*)(ws + plan.ranks);
  int32_t* inv_hi = (int32_t*)(ws + plan.inv[0]);
  int32_t* inv_lo = (int32_t*)(ws + plan.inv[1]);
  const dim3 gblk = seq_grid(nblk, B);
  uint32_t* tokmap = (uint32_t*)(cache + L->tokmap);
  int32_t* counters = (int32_t*)(cache + L->counters);
  const int nb4 = ceil_div(T, kBlkSort);
  const int ld = (T + 3) & ~3;               // 16-byte aligned rows of sorted keys
  const bool grouped = T > kMergeMaxT;       // sorted keys exceed one workgroup's LDS
  MergeArgs m;
  m.skeys = keys[0];
  m.sidx = sidx;
  m.scores = scores;
  m.ranks = ranks;
  m.ranks_out = ranks_out;
  m.sorted_asc = (float*)(cache + L->sorted);
  m.hicnt = segcnt;
  m.cnt = grouped ? keys[1] : nullptr;
  m.T = T; m.ld = ld; m.nblk = nb4; m.n_hi = n_hi; m.cap = L->cfg.capacity; m.B = B;
  m.ngrp = ceil_div(nb4, kMergeBlocks);
  k_rank_block_sort<<<seq_grid(nb4, B), kBlkThreads, 0, s>>>(scores, keys[0], sidx, segcnt, m.cnt, T,
                                                             ld, nb4, B);
  if (!grouped) {
    k_rank_merge<<<seq_grid(4 * nb4, B), 1024, 0, s>>>(m);
  } else {
    k_rank_merge_part<<<seq_grid(4 * nb4 * m.ngrp, B), 1024, 0, s>>>(m);
    k_rank_finish<<<seq_grid(4 * nb4, B), 1024, 0, s>>>(m);
  }
  int32_t* pos_hi = L->slot_pos[0] ? (int32_t*)(cache + L->slot_pos[0]) : nullptr;
  int32_t* pos_lo = L->slot_pos[1] ? (int32_t*)(cache + L->slot_pos[1]) : nullptr;
  k_rank_slots<kSortTile><<<gblk, 256, 0, s>>>(ranks, segcnt, tokmap, inv_hi, inv_lo, pos_hi, pos_lo,
                                               counters, T, n_hi, L->cfg.capacity, L->cap[0], L->cap[1],
                                               nblk, B);
  return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
