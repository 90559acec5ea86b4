// Internal declarations shared by the host entry points and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kSortTile = 1024;   // tokens per high-tier count segment and slot-scan workgroup
constexpr int kMaxSortLen = 1 << 18;   // longest ranked sequence (tokens)
constexpr int kMergeMaxT = 32768;      // up to this length: block sort + merge rank (keys in LDS)

inline int gcd_i(int a, int b) { while (b) { int t = a % b; a = b; b = t; } return a; }
inline int lcm_i(int a, int b) { return a / gcd_i(a, b) * b; }
inline int decode_chunk_kchan(const kvq_layout* L) {
  return lcm_i(lcm_i(L->cfg.k_block, 16), L->vnv);
}
constexpr int kWinChunk = 16;   // fp16-window tokens per decode workgroup
inline int kchan_nq(const kvq_layout* L, int T) {
  int kb = L->cfg.k_block;
  int n = (T - L->cfg.window) / kb;
  return n > 0 ? n * kb : 0;
}

// Number of decode chunks per unit for sequences of at most max_len tokens.
int decode_chunks(const kvq_layout* L, int max_len, int* nch0, int* nch1);

struct QuantWs {           // byte offsets inside the quantize workspace
  size_t keys[2], idx, segcnt, ranks, inv[2], total;   // keys[1]: partial counts (long sequences)
};
QuantWs quant_ws_plan(const kvq_layout* L, int T);

// Kernel launchers (return false when a launch failed).
// Writes one KV head's key and value channel orders (kD bytes each, passed
// by value) to dk and dv.
bool launch_write_order(uint8_t* dk, uint8_t* dv, const uint8_t* kbytes, const uint8_t* vbytes,
                        void* stream);

bool launch_rank_tiers(const kvq_layout* L, uint8_t* cache, const float* scores, int T, int n_hi,
                       int32_t* ranks_out, uint8_t* ws, const QuantWs& plan, void* stream);
bool launch_quantize_tiered(const kvq_layout* L, uint8_t* cache, const void* k, const void* v,
                            int64_t sb, int64_t st, int64_t sh, int T, int n_hi,
                            const uint8_t* ws, const QuantWs& plan, void* stream);
bool launch_quantize_kchan(const kvq_layout* L, uint8_t* cache, const void* k, const void* v,
                           int64_t sb, int64_t st, int64_t sh, int T, void* stream);
bool launch_append(const kvq_layout* L, uint8_t* cache, const void* k_new, const void* v_new,
                   const float* score_new, void* stream);
// Decode launchers return KVQ_ERR_WORKSPACE when the chunk split they chose
// needs more partials than the workspace holds, KVQ_ERR_LAUNCH when a launch
// failed.
kvq_status launch_decode(const kvq_layout* L, const uint8_t* cache, const void* q, float scale,
                         int max_len, void* out, uint8_t* ws, void* stream, float* mass = nullptr);
// Workspace of a decode (partials), plus, with the token mass, the pools'
// raw scores and the per-head (max, sum) after the merge.
size_t decode_ws_bytes(const kvq_layout* L, int max_len, bool mass);
// Partial bytes written with the split launch_decode chooses (<= decode_ws_bytes).
size_t decode_ws_used(const kvq_layout* L, int max_len);
// Decode with its partials in the library's fixed device array (at most
// kNoAllocScratchBytes; KVQ_ERR_WORKSPACE beyond it); allocates nothing.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
kvq_status launch_decode_noalloc(const kvq_layout* L, const uint8_t* cache, const void* q, float scale,
                                 int max_len, void* out, void* stream);

// One tier pool of the matrix-core decode kernel.
struct PoolArgs {
  const int32_t* counters;
  const uint16_t* q;
  float* part;
  const uint32_t* kwords;
  const uint32_t* kmeta;
  const uint32_t* vwords;
  const uint32_t* vmeta;
  int pool, Hkv, tiles, vrows, nch_total, part_off;
  int chunk;          // slots per workgroup at full capacity (sets the grid; the kernel
                      // splits the filled slots evenly over gridDim.x chunks)
  float c;            // softmax scale * log2(e)
  float* raw;         // or null: log2-domain scores out, [unit][head][cap_p]
  int cap_p;          // slots of this pool
  const uint8_t* korder = nullptr;   // [Hkv][128] stored key channel order: q is read through it
  const int32_t* spos = nullptr;     // pre-RoPE keys: [B][cap_p] token position of each slot
  float rope_theta = 0.0f;           // rotary base (with spos)
};
// Slots per workgroup for one pool so that the grid fills the chip about once
// (uses the kernel's occupancy; falls back to 8 macro tiles).
int decode_pool_chunk(int L, int G, int U, int slots_per_unit, bool rope = false);
// The device's CU count (cached per device).
int device_cu_count();
// Slots per chunk (whole macro tiles) so that U units' chunks make about one
// round of a kernel resident at blocks_per_cu workgroups per CU.
int chunk_for_one_round(int L, int U, int slots_per_unit, int blocks_per_cu);
bool launch_decode_pool(int L, const PoolArgs& a, int G, int nch, int U, void* stream);
// Both tier pools in one launch: chunks per unit for a level pair that has a
// one-launch kernel (0: none, launch one kernel per pool), and the launch
// (a0.part, a0.nch_total and a0.counters serve both; partial c per chunk).
int decode_pair_chunks(int L0, int L1, int G, int U, int slots0, int slots1);
bool launch_decode_pair(int L0, int L1, int G, const PoolArgs& a0, const PoolArgs& a1, int nch, int U,
                        void* stream);
// One tier pool of the multi-query kernel: four query tokens per workgroup.
struct PoolMqArgs {
  const int32_t* counters;
  const uint16_t* q;            // [B][M][Hq][D]
  float* part;                  // [unit][query group][chunk][16 rows][4 + D]
  const uint32_t* kwords;
  const uint32_t* kmeta;
  const uint32_t* vwords;
  const uint32_t* vmeta;
  int pool, Hkv, M, nqg, tiles, vrows, nch_total, part_off;
  int chunk;          // slots per workgroup at full capacity (sets the grid; the kernel
                      // splits the filled slots evenly over gridDim.x chunks)
  float c;            // softmax scale * log2(e)
  const uint8_t* korder = nullptr;   // [Hkv][128] stored key channel order: q is read through it
};
// Attention of M query tokens per sequence over a tiered cache (output and
// log-sum-exp); KVQ_ERR_UNSUPPORTED when the mode is not tiered.
kvq_status launch_decode_mq(const kvq_layout* L, const uint8_t* cache, const void* q, int M, float scale,
                            int max_len, void* out, float* lse, uint8_t* ws, void* stream);
size_t decode_mq_ws_bytes(const kvq_layout* L, int M, int max_len);
// Read-stream probe (every byte once, 16-byte loads) over nwg workgroups.
bool launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int nwg, void* stream);
// Matrix-core decode of a per-channel-key cache: nch0 quantized chunks and
// nwch fp16-window chunks per unit in one launch; false when the
// configuration is not the one it is built for.
bool launch_decode_kchan_mfma(const kvq_layout* L, const uint8_t* cache, const void* q, float c,
                              float* part, int nch0, int nwch, int nch_total, void* stream);

}  // namespace kvq
