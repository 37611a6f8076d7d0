// Internal helpers shared by the HIP kernels of libtv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tv.h"

namespace tv {

// ---------------------------------------------------------------- element types
// bf16 values travel as raw 16-bit patterns; arithmetic is always fp32.

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (gfx950 converts with v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- wave64 reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = (uint32_t)__shfl((int)lo, src, 64);
  hi = (uint32_t)__shfl((int)hi, src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Tiles of one (sequence, KV head) that a contiguous pool keeps next to each other.
constexpr int kTileRun = 16;

// Element offset of tile t (entries 64t .. 64t+63) of (sequence b, KV head g) in a
// level's K or V^T pool (both hold 64*d elements per tile).  Paged pool: tile g of the
// physical page `page` (the caller reads page_table[b][t]), pages being the Hkv heads'
// tiles of one (sequence, 64 entries).  Contiguous pool of capacity cap (T = cap/64
// tiles per (b, g)): the tiles come in runs of kTileRun consecutive tiles of one (b, g);
// the runs covering tiles [R*q, R*q + R) of every (b, g) are side by side, in (b, g)
// order, run range after run range; the last T mod R tiles of each (b, g) follow, (b, g)
// after (b, g).  The workgroups streaming every sequence's prefix at once thus read
// within one window of memory rather than at a fixed stride of one sequence's pool,
// while each still reads runs of 256 KB (K) in order.
__device__ __forceinline__ size_t tile_offset(bool paged, int page, int cap, int B, int Hkv, int d, int b, int g,
                                              int t) {
  size_t tile;
  if (paged) {
    tile = (size_t)page * Hkv + g;
  } else {
    const int T = cap / 64, full = T / kTileRun;  // complete run ranges
    const int q = t / kTileRun, w = t - q * kTileRun;
    tile = q < full ? (((size_t)q * B + b) * Hkv + g) * kTileRun + w
                    : (size_t)full * B * Hkv * kTileRun + ((size_t)b * Hkv + g) * (T - full * kTileRun) + w;
  }
  return tile * 64 * d;
}

// Physical page of tile t of sequence b in a level (0 for a contiguous pool); false if the
// page-table entry is outside [0, num_pages).
__device__ __forceinline__ bool tile_page(const tv_level& L, int b, int t, int* page) {
  if (L.page_table == nullptr) {
    *page = 0;
    return true;
  }
  const int p = L.page_table[(size_t)b * L.pages_per_seq + t];
  *page = p;
  return p >= 0 && p < L.num_pages;
}

// bits of the nodes 0..D-1 of a tree
__device__ __forceinline__ uint64_t node_mask(int D) { return D >= 64 ? ~0ull : ((1ull << D) - 1ull); }

// committed entries of a level, never beyond the pool's capacity
__device__ __forceinline__ int level_count(const int32_t* n, int b, int cap) {
  return max(0, min(n[b], cap));
}

// log2(e): scores are kept in base-2 units (s * log2(e) / sqrt(d)) so exp2 can be used.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- launch arguments

struct AttnArgs {
  int B, D, Hq, Hkv, d, G, R;        // R = G * D query rows per (sequence, KV head)
  int dtype;                         // tv_dtype
  int n_levels;
  int C[TV_MAX_LEVELS], cap[TV_MAX_LEVELS];
  const void* pk[TV_MAX_LEVELS];     // pools, K row-major
  const void* pvt[TV_MAX_LEVELS];    // pools, V transposed
  const int32_t* pn[TV_MAX_LEVELS];
  const int32_t* pt[TV_MAX_LEVELS];  // page tables (NULL: contiguous pool)
  int ppseq[TV_MAX_LEVELS], npages[TV_MAX_LEVELS];
  const float* open_k[TV_MAX_LEVELS];
  const float* open_v[TV_MAX_LEVELS];
  const void* tail_k;
  const void* tail_v;
  const int32_t* P;
  const void* q;
  const void* k_tree;
  const void* v_tree;
  const uint64_t* anc;                // [B][anc_ld]: the first D entries of a row are this tree's
  const int32_t* depth;               // [B][anc_ld]
  int anc_ld;                         // row length of anc and depth (>= D)
  const int32_t* seq_err;            // may be null
  void* out;
  float* lse;                        // may be null
  tv_scratch scratch;                // entries may be null
  int build_scratch;
  // Prefix-stream partition.  A unit is one (sequence, KV head, block of unit_rows query
  // rows); its prefix is `tmax` 64-entry chunks long (a bound from the pool capacities;
  // chunks past a sequence's committed entries are empty).  The units' chunks, laid end
  // to end, are cut into `parts` slices of equal length to within one chunk (slice_begin),
  // one workgroup each.  A
  // slice touches a run of consecutive units, and consecutive slices share at most one
  // unit, so (slice p, unit u) pairs are numbered uniquely by p + u (< parts + units - 1):
  // the partial of that pair is the workspace's row block p + u (partial_row()).
  int unit_rows;                     // query rows of a unit: 64, or 128 for the 8-wave MFMA instance
  int row_blocks;                    // RB = ceil(R / unit_rows)
  int tmax;                          // chunks per unit
  int units;                         // B * Hkv * RB (units * tmax < 2^31)
  int parts;                         // workgroups of the prefix stream
  int total;                         // units * tmax chunk slots
  int idx32;                         // parts * total < 2^32: slice arithmetic in 32 bits
  int nt_partials;                   // partials written and read with the nontemporal hint
  int merge_nmax;                    // a bound on the slices of one unit (the merge's shape)
  int fused_tree;                    // the MFMA prefix kernel also attends to the raw tail and
                                     // the tree chunk, and writes whole units' rows itself
  int tree_tiles;                    // 16-entry tiles of that chunk: 1, 2 or 4
  int fold_scratch;                  // MFMA prefix kernel: its first fold_scratch workgroups
                                     // build the scratch pad (one per (sequence, node)), the
                                     // prefix stream's `parts` workgroups follow
  int pad_after;                     // the fold_scratch workgroups come after the stream's instead
                                     // (they then fill the slots of the first slices to finish)
  float* ws_o;                       // [parts + units - 1][unit_rows][d] (unused if no unit is split)
  float2* ws_ml;                     // [parts + units - 1][unit_rows] (running max in log2 units, sum)
  float scale_log2;                  // log2(e) / sqrt(d)
};

// Workspace row of the partial that slice `part` leaves for local row `lrow` (0 ..
// unit_rows-1) of unit u.
__device__ __forceinline__ size_t partial_row(const AttnArgs& a, long long part, long long u, int lrow) {
  return (size_t)(part + u) * a.unit_rows + lrow;
}

// The prefix of a (sequence, KV head) is streamed as 64-entry chunks: level 0's
// ceil(n0/64) chunks, then level 1's.  Slices take runs of whole chunks, so a
// chunk never straddles two levels and always starts 64-aligned in its pool.
// chunk c of a sequence's concatenated pools -> (level, first entry, entry count)
__device__ __forceinline__ void chunk_entries(int n0, int T0, int n1, int c, int* lvl,
                                              int* e0, int* cnt) {
  if (c < T0) {
    *lvl = 0;
    *e0 = c * 64;
    *cnt = min(64, n0 - c * 64);
  } else {
    *lvl = 1;
    *e0 = (c - T0) * 64;
    *cnt = min(64, n1 - (c - T0) * 64);
  }
}

// Slice p of the prefix stream is the chunks [p * total / parts, (p + 1) * total / parts)
// of the units' chunks laid end to end (1 <= parts <= total < 2^31): slice lengths differ by
// at most one chunk, so every workgroup of the one round has the same work to within a
// chunk.  In 32-bit arithmetic when parts * total < 2^32 (idx32, set on the host).
__device__ __forceinline__ int slice_begin(const AttnArgs& a, int p) {
  if (a.idx32) return (int)((uint32_t)p * (uint32_t)a.total / (uint32_t)a.parts);
  return (int)((long long)p * a.total / a.parts);
}
// the slice holding chunk x (the largest p with slice_begin(p) <= x)
__device__ __forceinline__ int slice_of(const AttnArgs& a, int x) {
  if (a.idx32) return (int)(((uint32_t)x * (uint32_t)a.parts + (uint32_t)a.parts - 1u) / (uint32_t)a.total);
  return (int)(((long long)x * a.parts + a.parts - 1) / a.total);
}
// first workgroup whose slice touches unit u, and how many workgroups touch it
__device__ __forceinline__ int unit_first_part(const AttnArgs& a, int u) { return slice_of(a, u * a.tmax); }
__device__ __forceinline__ int unit_part_count(const AttnArgs& a, int u) {
  return slice_of(a, u * a.tmax + a.tmax - 1) - slice_of(a, u * a.tmax) + 1;
}

}  // namespace tv
