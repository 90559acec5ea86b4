// Compile-time tiling of the matrix-core decode kernel for one grid of L
// levels (shared by the kernel and by the host's workspace sizing).
#pragma once

namespace kvq {

__host__ __device__ constexpr int cpw(int L) {
  // max{n : L^n <= 2^32}
  unsigned long long p = 1;
  int n = 0;
  while (p * (unsigned long long)L <= (1ull << 32)) {
    p *= (unsigned long long)L;
    ++n;
  }
  return n;
}

// Value word rows owned by one lane group per macro tile: the slots of a
// macro tile (4 * R * nv) must be a whole number of 16-slot key tiles; among
// R in {1, 2, 4} pick the one with the least padding of the lane's slot run
// (R * nv) to the 8-slot granularity of the matrix instruction.
__host__ __device__ constexpr int macro_rows(int nv) {
  int best = 4, waste_best = 1 << 30;
  for (int R = 1; R <= 4; R *= 2) {
    if ((R * nv) % 4 != 0 || 4 * R * nv > 256) continue;
    int slots = R * nv;
    int pad = ((slots + 7) / 8) * 8 - slots;
    int waste = pad * 64 / slots;   // per-mille-ish, lower is better
    if (waste < waste_best) { waste_best = waste; best = R; }
  }
  return best;
}

template <int L>
struct Tiling {
  static constexpr int NV = cpw(L);                    // codes per word
  static constexpr int KW = (128 + NV - 1) / NV;       // key words per row
  static constexpr int KWL = (KW + 3) / 4;             // key words per lane (max)
  static constexpr int R = macro_rows(NV);             // value word rows per lane group
  static constexpr int RUN = R * NV;                   // slots per lane group per macro tile
  static constexpr int MT = 4 * RUN;                   // slots per macro tile
  static constexpr int KT = MT / 16;                   // key tiles per macro tile
  static_assert(MT % 16 == 0, "macro tile must hold whole key tiles");
};

// Slots of one macro tile for a pool with L levels (the unit of decode work).
__host__ __device__ constexpr int macro_tile_slots(int L) {
  return 4 * macro_rows(cpw(L)) * cpw(L);
}

}  // namespace kvq
