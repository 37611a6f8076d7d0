// Branch-aware verify attention: bf16 MFMA kernel (gfx950).
// TSD-V4 §3.1 (each candidate attends to the accepted context and to the ancestors
// on its own branch only), §2.2 (the context is the multi-resolution compressed
// history), §2.1 / §5.3 (verification of many candidates is memory-bound at small
// batch: the prefix is read once for all G*D query rows of a KV head).
//
// A unit is one (sequence, KV head, block of 16 * NW query rows): 64-row units in 4-wave
// workgroups (two per CU), or, when a KV head has more than 64 rows (G * D > 64),
// 128-row units in 8-wave workgroups (one per CU) so that every row of the head shares
// one stream.  The units' prefixes, cut into 64-entry chunks and laid end to end, are
// split into slices of equal length to within one chunk, one persistent workgroup each
// (one round on the GPU); 16
// query rows per wave (rows r = node * G + head-in-group).  Per 64-entry chunk:
//   1. the K chunk (64 x 128, row-major) and the V^T tile (128 x 64; the V pool is
//      stored transposed per 64-entry tile) are each one contiguous 16 KB block,
//      loaded with 16-byte coalesced loads into registers two chunks ahead (two
//      register buffers), all issued back to back, then written to LDS (straight
//      copies, padded rows), into one of two LDS buffers by chunk parity, so that a
//      chunk costs one barrier: the buffer written for chunk c was last read for chunk
//      c - 2, which every wave finished before the barrier after chunk c - 1's stores;
//   2. S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the K chunk is the A operand
//      (16 entries x 32 channels per lane group), Q^T the B operand kept in
//      registers; the accumulator gives each lane one query row and 4 entries per
//      16-entry tile;
//   3. online softmax in base-2 units: the row max is combined across the four
//      lane groups by two xor shuffles; each lane keeps its own partial sum; the
//      accumulators are rescaled only when some row's maximum moved;
//   4. O^T += V^T P^T with the same MFMA: the transposed V chunk is the A operand
//      (16 channels x 32 entries), stored in LDS in the entry order the softmax
//      lanes hold so each operand is one conflict-free 16-byte read; P^T (bf16)
//      is the B operand straight from registers, and the accumulator again gives
//      each lane its own query row, so the rescale needs no data movement.
// The workgroup whose slice holds a unit's first chunk also attends to one more chunk
// built from the finest level's raw tail and the tree tokens of the unit's KV head;
// there a row sees the tail and exactly the nodes of its own chain (bits of the
// node's ancestor mask), everything else is excluded by selection.  If that
// workgroup's slice covers the whole unit it normalises and writes the output rows and
// their LSE; otherwise every workgroup of the unit writes a partial (running max, sum,
// unnormalised output) for the merge kernel.
#include "scratch_pad.h"
#include "tv_launch.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int kDH = 128;        // head dim handled by this kernel
constexpr int kChunk = 64;      // entries per chunk
// LDS layouts, chosen by measuring ds_read_b128 on gfx950 (64 banks): under load a row
// stride of an odd number of 16-byte units (272 B for K, 144 B for V^T) costs 1.6x the
// cycles of a conflict-free read, an even number (288 B) or an XOR swizzle does not.
constexpr int kKStr = kDH * 2 + 32;      // LDS bytes per K row (padded to 18 units of 16 B)
constexpr int kVStr = kChunk * 2;        // LDS bytes per V^T row (unpadded, 16-byte units swizzled)
// the V area also holds the tree chunk's V rows, entry-major with the K row stride
constexpr int kVBytes = kDH * kVStr > kChunk * kKStr ? kDH * kVStr : kChunk * kKStr;
constexpr int kLdsBytes = kChunk * kKStr + kVBytes;
// LDS slot of entry e (0..63) within a V^T row.  The P^T operand of the PV product gives
// lane group grp the entries 32h + 4grp + {0..3} and 32h + 16 + 4grp + {0..3} of k-step h;
// storing them at slots 32h + 8grp + {0..7} makes each operand one 16-byte LDS read.
__device__ __forceinline__ int v_slot(int e) {
  return (e & 32) + 8 * ((e & 15) >> 2) + 4 * ((e >> 4) & 1) + (e & 3);
}
// Byte offset of slot s of V^T row r: 16-byte unit s/8 of the row is stored at unit
// (s/8) ^ (r & 7), so the 16 rows one operand read touches fall in distinct bank groups.
__device__ __forceinline__ int vt_byte(int r, int s) {
  return r * kVStr + ((((s >> 3) ^ (r & 7)) << 4) | ((s & 7) << 1));
}
// Maximum of v over lanes l and l ^ 16, and then over l ^ 32: gfx950's permlane swaps
// (v_permlane16_swap / v_permlane32_swap, vector ALU) return the two 16-lane (32-lane)
// halves of each pair, so the larger of the two results is the pair's maximum in every
// lane -- no trip through the LDS crossbar as for a general shuffle.
// Maximum of two scores as v_maximum3_f32 (NaN-propagating): fmaxf's IEEE maxNum makes the
// compiler quiet each matrix-core result first (one more instruction per score).  A NaN
// score would poison its row either way (its exp2 is NaN); excluded entries are -inf by
// selection before any maximum.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax2(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
// One 16-byte piece of a pool tile, loaded with the nontemporal hint (the `nt` cache
// policy): a launch reads each tile exactly once, so the caches need not keep it.  On
// MI355X this lifts a plain read of HBM from about 6.3 to about 7.1 TB/s and this
// kernel's stream by about 10%.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const char* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
}  // namespace

// 16 KB of zeros: the load target of chunk slots past the end of a unit's stream.  Every
// slot's loads are then issued unconditionally, so the wait before a chunk is written to
// LDS counts exactly the loads issued after it and the next chunk stays in flight.
static __device__ __attribute__((aligned(256))) uint4 g_zero_chunk[1024];

// At most 256 VGPRs: two workgroups per CU, each with two chunks (64 KB) in flight.  TT is
// the number of 16-entry tiles the tail + tree chunk takes (its registers are sized by it);
// PAGED selects paged pools (a page-table read per chunk) over contiguous ones.
template <int NW, int TT, bool PAGED>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void k_attn_mfma(AttnArgs a) {
  static_assert(NW == 4 || NW == 8, "4 waves (64-row units, two workgroups per CU) or 8 (128-row units, one)");
  constexpr int NT = NW * 64;
  constexpr int kUnitRows = 16 * NW;          // query rows of a unit: 16 per wave
  constexpr int PER = (1024 + NT - 1) / NT;   // K pieces (and V pieces) per thread
  constexpr bool kFull = 1024 % NT == 0;
  static_assert(TT >= 1 && TT <= 4, "the tail + tree chunk is at most 64 entries");
  constexpr int TPER = (TT * 256 + NT - 1) / NT;  // its K (and V) pieces per thread
  constexpr bool kTFull = (TT * 256) % NT == 0;
  __shared__ __attribute__((aligned(16))) char smem[2 * kLdsBytes];  // two chunk buffers (two workgroups fit a CU)
  __shared__ uint64_t anc_s[TV_MAX_D];
  char* Ks = smem;
  char* Vs = smem + kChunk * kKStr;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  // scratch-pad workgroups (uniform; 256 threads): the first fold_scratch workgroups, or,
  // with pad_after, the last ones (dispatched as the stream's workgroups retire)
  const int pad0 = a.pad_after ? a.parts : 0;
  if (NW == 4 && (int)blockIdx.x >= pad0 && (int)blockIdx.x < pad0 + a.fold_scratch) {
    const int item = blockIdx.x - pad0;
    const int sb = item / a.D;
    scratch_node<uint16_t, 4>(a, sb, item - sb * a.D, (ScratchLds*)smem);  // (4: no spill beside the stream's registers)
    return;
  }
  const int part = a.pad_after ? (int)blockIdx.x : (int)blockIdx.x - a.fold_scratch;  // this workgroup's slice
  // two chunks of loads in flight (8 waves: a third measured nothing, the LDS reads of 8
  // waves per chunk bound that instance)
  uint4 kpa[PER], vpa[PER], kpb[PER], vpb[PER];

  // this workgroup's slice of the units' chunks, laid end to end
  int cg = slice_begin(a, part);
  const int cend = slice_begin(a, part + 1);
  while (cg < cend) {
    const int u = cg / a.tmax;
    const int c_first = cg - u * a.tmax;
    const int c_last = min(a.tmax, cend - u * a.tmax);
    const bool whole_unit = c_first == 0 && c_last == a.tmax;  // no other workgroup touches it
    const int rb = u % a.row_blocks;
    const int g = (u / a.row_blocks) % a.Hkv;
    const int b = u / (a.row_blocks * a.Hkv);
    const size_t bg = (size_t)b * a.Hkv + g;

    // Q^T operand: lane (n16, grp), k-step ks holds Q[row][32ks + 8grp .. +7]
    const int row = rb * kUnitRows + w * 16 + n16;
    const int node = row < a.R ? row / a.G : 0;
    const int head = g * a.G + (row - node * a.G);
    const bool wave_has_rows = rb * kUnitRows + w * 16 < a.R;  // wave-uniform
    bf16x8 qop[4];
    {
      const uint16_t* q = (const uint16_t*)a.q;
      if (row < a.R) {
        const uint16_t* qr = q + (((size_t)b * a.D + node) * a.Hq + head) * kDH;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = *(const bf16x8*)(qr + 32 * ks + 8 * grp);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qop[ks] = bf16x8{};
      }
    }

    // the sequence's error code, committed counts and prefix length in one round trip:
    // lane 0 loads seq_err[b], lane 1 + l the count of level l, lane 3 P[b]
    int uval = 0;
    {
      const int32_t* src = nullptr;
      if (lane == 0) src = a.seq_err != nullptr ? a.seq_err + b : nullptr;
      else if (lane == 1) src = a.n_levels > 0 ? a.pn[0] + b : nullptr;
      else if (lane == 2) src = a.n_levels > 1 ? a.pn[1] + b : nullptr;
      else if (lane == 3) src = a.P + b;
      if (src != nullptr) uval = *src;
    }
    const bool live = a.seq_err == nullptr || __builtin_amdgcn_readlane(uval, 0) == TV_SEQ_OK;
    const int n0 = a.n_levels > 0 ? max(0, min(__builtin_amdgcn_readlane(uval, 1), a.cap[0])) : 0;
    const int n1 = a.n_levels > 1 ? max(0, min(__builtin_amdgcn_readlane(uval, 2), a.cap[1])) : 0;
    const int Pb = __builtin_amdgcn_readlane(uval, 3);
    const int T0 = (n0 + 63) / 64, T1 = (n1 + 63) / 64;
    const int c_lo = c_first;
    const int c_hi = live ? min(c_last, T0 + T1) : c_first;

    // Pieces: 1024 16-byte pieces of K (row p/16, column p%16) and 1024 of V^T (row p/8,
    // column p%8) per chunk; thread tid takes pieces tid, tid + NT, ...  A chunk is
    // 64-aligned in its pool and a pool's capacity is a multiple of 64, so all 64 entries
    // of a chunk are in bounds: every piece is loaded unconditionally (no data-dependent
    // code between the loads, so they are all in flight together) and entries past the
    // committed count are zeroed by selection when the chunk is written to LDS.
    // Slots c >= c_hi (past the unit's stream) read the zero block, and so does a chunk of a
    // paged pool whose page id is out of range.  `pid` is the chunk's page (paged pools).
    // Contiguous pools: tile_offset's placement with its per-unit parts worked out once, so
    // that a chunk's tile costs a compare, a shift and a multiply-add (scalar) rather than
    // the full computation: tile t of level l (t < 16 * full_l) is run0 + (t / 16) * run_step
    // + t % 16, a tile of the last incomplete run is tail0_l + t - 16 * full_l.
    const int bgi = b * a.Hkv + g;
    const int run_step = a.B * a.Hkv * kTileRun;
    const int full0 = a.cap[0] / 64 / kTileRun, full1 = a.n_levels > 1 ? a.cap[1] / 64 / kTileRun : 0;
    const int tail00 = full0 * run_step + bgi * (a.cap[0] / 64 - full0 * kTileRun);
    const int tail01 = a.n_levels > 1 ? full1 * run_step + bgi * (a.cap[1] / 64 - full1 * kTileRun) : 0;
    auto load_chunk = [&](int c, int pid, uint4 (&kpre)[PER], uint4 (&vpre)[PER]) {
      const char* kb = (const char*)g_zero_chunk;
      const char* vb = kb;
      if (c < c_hi) {  // uniform
        const bool l1 = c >= T0;
        const int t = l1 ? c - T0 : c;  // the chunk's tile within its level
        if (!PAGED) {
          const int full = l1 ? full1 : full0;
          const int tile = t < full * kTileRun ? bgi * kTileRun + (t / kTileRun) * run_step + t % kTileRun
                                               : (l1 ? tail01 : tail00) + t - full * kTileRun;
          const size_t off = (size_t)tile * (64 * kDH * 2);
          kb = (const char*)(l1 ? a.pk[1] : a.pk[0]) + off;    // K rows
          vb = (const char*)(l1 ? a.pvt[1] : a.pvt[0]) + off;  // V^T tile
        } else if (pid >= 0 && pid < (l1 ? a.npages[1] : a.npages[0])) {
          const size_t off = tile_offset(true, pid, 0, a.B, a.Hkv, kDH, b, g, t) * 2;
          kb = (const char*)(l1 ? a.pk[1] : a.pk[0]) + off;
          vb = (const char*)(l1 ? a.pvt[1] : a.pvt[0]) + off;
        }
      }
      // piece p = tid + x * NT at byte 16p of each tile (K rows are 256 B, V^T rows 128 B):
      // a uniform base per x plus the thread's own 32-bit offset
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int p = tid + x * NT;
        if (kFull || p < 1024) {
          kpre[x] = load_stream16(kb + x * NT * 16 + (uint32_t)tid * 16);
          vpre[x] = load_stream16(vb + x * NT * 16 + (uint32_t)tid * 16);
        }
      }
    };
    auto store_chunk = [&](int cnt, uint4 (&kpre)[PER], uint4 (&vpre)[PER], int buf) {
      if (cnt < 64) {  // partial chunk (uniform): zero what lies past the committed count
#pragma unroll
        for (int x = 0; x < PER; ++x) {
          const int p = tid + x * NT;
          if (kFull || p < 1024) {
            const uint32_t krow_ok = (p >> 4) < cnt ? 0xffffffffu : 0u;
            kpre[x].x &= krow_ok; kpre[x].y &= krow_ok; kpre[x].z &= krow_ok; kpre[x].w &= krow_ok;
            const int keep = cnt - (p & 7) * 8;  // committed entries among this piece's 8
            vpre[x].x &= (keep > 0 ? 0x0000ffffu : 0u) | (keep > 1 ? 0xffff0000u : 0u);
            vpre[x].y &= (keep > 2 ? 0x0000ffffu : 0u) | (keep > 3 ? 0xffff0000u : 0u);
            vpre[x].z &= (keep > 4 ? 0x0000ffffu : 0u) | (keep > 5 ? 0xffff0000u : 0u);
            vpre[x].w &= (keep > 6 ? 0x0000ffffu : 0u) | (keep > 7 ? 0xffff0000u : 0u);
          }
        }
      }
      // piece p = tid + x * NT: K row p / 16, 16-byte unit p % 16; V^T channel row p / 8,
      // entries 8 (p % 8) .. +7, whose two halves go to their slots in the lane order of the
      // P^T operand (see v_slot).  NT is a multiple of 128, so the LDS address of piece x is
      // thread tid's address plus a constant (row r + NT/8 has the swizzle of row r), which
      // the stores carry as an immediate offset instead of a register per piece.
      char* k_st = Ks + buf * kLdsBytes + (tid >> 4) * kKStr + (tid & 15) * 16;
      char* v_st0 = Vs + buf * kLdsBytes + vt_byte(tid >> 3, v_slot((tid & 7) * 8));
      char* v_st1 = Vs + buf * kLdsBytes + vt_byte(tid >> 3, v_slot((tid & 7) * 8 + 4));
#pragma unroll
      for (int x = 0; x < PER; ++x) {
        const int p = tid + x * NT;
        if (kFull || p < 1024) {
          *(uint4*)(k_st + x * (NT / 16) * kKStr) = kpre[x];
          *(uint2*)(v_st0 + x * (NT / 8) * kVStr) = make_uint2(vpre[x].x, vpre[x].y);
          *(uint2*)(v_st1 + x * (NT / 8) * kVStr) = make_uint2(vpre[x].z, vpre[x].w);
        }
      }
    };

    f32x4 oacc[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // Attend to the chunk in LDS.  hide(t, i) is true for the scores to leave out (entry
    // 16t + 4grp + i of this lane's row); it is only evaluated when `masked`.
    auto attend = [&](bool masked, auto hide, int buf) {
      const char* Kb = Ks + buf * kLdsBytes;
      const char* Vb = Vs + buf * kLdsBytes;
      // S^T tiles: sacc[t] lane (n16, grp) = S[row n16][entry 16t + 4grp + i].  The K
      // operands of tile t + 1 are read from LDS into a second set of registers before
      // tile t's products, which lets the compiler keep several reads in flight (each wait
      // covers only the older reads) instead of waiting for every read before its product:
      // the LDS latency then overlaps the matrix cores instead of adding up read by read.
      f32x4 sacc[4];
      bf16x8 kop[2][4];
      auto read_k = [&](int t, bf16x8 (&dst)[4]) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) dst[ks] = *(const bf16x8*)(Kb + (16 * t + n16) * kKStr + (32 * ks + 8 * grp) * 2);
      };
      read_k(0, kop[0]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < 3) read_k(t + 1, kop[(t + 1) & 1]);
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[t & 1][ks], qop[ks], sacc[t], 0, 0, 0);
      }
      // Online softmax in base-2 units.  The scale is applied inside the exponent (one
      // fma per score); the row max is taken on raw scores (scale > 0).
      if (masked) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (hide(t, i)) sacc[t][i] = -INFINITY;
      }
      float mx = fmax2(fmax2(fmax2(sacc[0][0], sacc[0][1]), fmax2(sacc[0][2], sacc[0][3])),
                       fmax2(fmax2(sacc[1][0], sacc[1][1]), fmax2(sacc[1][2], sacc[1][3])));
      mx = fmax2(mx, fmax2(fmax2(fmax2(sacc[2][0], sacc[2][1]), fmax2(sacc[2][2], sacc[2][3])),
                           fmax2(fmax2(sacc[3][0], sacc[3][1]), fmax2(sacc[3][2], sacc[3][3]))));
      mx = max_xor16_32(mx);
      // a row with every score hidden keeps its state (its max stays -inf, p = 0)
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      // rows whose running max moved rescale their accumulators; skipped when none moved
      if (__ballot(m_new > m_run) != 0ull) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
      }
      m_run = m_new;
      bf16x8 pop[2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // exp2 of a non-positive argument; results below the normal range are flushed,
          // which cannot change a probability that is summed with at least one 1.0
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][i], a.scale_log2, -m_use));
          l_run += p;
          pop[t >> 1][(t & 1) * 4 + i] = (__bf16)p;
        }
      }
      // O^T += V^T P^T; k-step h: slots 32h + 8grp .. +7 hold entries 32h + 4grp + {0..3}
      // and 32h + 16 + 4grp + {0..3}
      // (the V^T operands of channel tiles 2j + 2, 2j + 3 are read into a second set of
      // registers before those of 2j, 2j + 1 are used, as for K)
      bf16x8 vop[2][4];
      auto read_v = [&](int j, bf16x8 (&dst)[4]) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          dst[x] = *(const bf16x8*)(Vb + vt_byte(16 * (2 * j + (x >> 1)) + n16, 32 * (x & 1) + 8 * grp));
      };
      read_v(0, vop[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < 3) read_v(j + 1, vop[(j + 1) & 1]);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int dt = 2 * j + (x >> 1);
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[j & 1][x], pop[x & 1], oacc[dt], 0, 0, 0);
        }
      }
    };

    // Page ids of paged pools: chunk c's page is read from the page table one step before
    // its loads are issued, and ahead of that step's own chunk loads, so waiting for it
    // never waits for chunk data.  Exactly one read per step (slots past the stream read
    // the zero block), so the wait before a chunk counts the same loads on every path.
    // Contiguous pools read nothing.
    auto load_pid = [&](int c) -> int {
      if (!PAGED) return 0;
      const int32_t* src = (const int32_t*)g_zero_chunk;
      if (c < c_hi) {  // uniform
        const bool l1 = c >= T0;
        src = (l1 ? a.pt[1] : a.pt[0]) + (size_t)b * (l1 ? a.ppseq[1] : a.ppseq[0]) + (l1 ? c - T0 : c);
      }
      return *src;
    };
    int pid_next = 0;  // page of the chunk the next step loads

    // One prefix chunk slot: if c is in the stream, write its chunk to LDS; refill the
    // slot's registers with chunk c + 2 (always issued, so that it is in flight with
    // chunk c + 1's loads); attend.
    auto step = [&](int c, uint4 (&kpre)[PER], uint4 (&vpre)[PER], int buf) {
      const bool have = c < c_hi;  // uniform
      int cnt = 0;
      if (have) {
        int lvl, e0;
        chunk_entries(n0, T0, n1, c, &lvl, &e0, &cnt);
        // (LDS buffer buf was last read for chunk c - 2: every wave finished that before
        // the barrier that followed chunk c - 1's stores)
        store_chunk(cnt, kpre, vpre, buf);
        __syncthreads();
      }
      const int pid = pid_next;
      pid_next = load_pid(c + 3);
      load_chunk(c + 2, pid, kpre, vpre);
      if (!have || !wave_has_rows) return;
      // The wave's matrix-core and softmax work on the chunk runs at a raised issue
      // priority (4-wave instance): on a SIMD shared by two workgroups the other wave's LDS
      // stores and next loads then fill the gaps of this critical chain instead of
      // delaying it (B = 64, 32768-token prefix: 380 -> 368 us per call under the
      // five-step warm-up; the 8-wave instance measured no gain).
      if (NW == 4) __builtin_amdgcn_s_setprio(1);
      attend(cnt < 64, [&](int t, int i) { return 16 * t + 4 * grp + i >= cnt; }, buf);
      if (NW == 4) __builtin_amdgcn_s_setprio(0);
    };

    // The unit's tail + chain chunk, attended first: entries [0, rr) are the finest level's
    // raw tail (visible to every row), entries rr + j the tree node j of this KV head
    // (visible to the rows of node i iff bit j of anc[i] is set).  Built by the workgroup
    // holding the unit's first chunk.  Its global loads are issued before those of the
    // first two prefix chunks, so that waiting for them leaves the prefix loads in flight
    // while the chunk is attended (pieces of rows past the tail and the tree read node 0
    // and are zeroed by selection).  Scores use the MFMA as below; the PV part runs on the
    // vector ALU, each lane adding only the entries its row sees, so a value a row does
    // not see is never multiplied (not even by a zero probability).
    const bool tree_here = a.fused_tree && c_first == 0 && live;
    const int C0 = a.n_levels > 0 ? a.C[0] : 1;
    // Beyond its own loads (issued here) the stage reads only kernel arguments (constant
    // level indices) and LDS: a vector load issued after the prefix loads would make its
    // wait also wait for those.
    const int rr = tree_here && C0 > 1 ? Pb % C0 : 0;
    const int ne = rr + a.D;  // <= 16 * TT
    char* Vr = Vs;  // V rows, entry-major, same padded stride as K (fits in the V^T area)
    uint4 tkp[TPER], tvp[TPER];
    uint64_t anc_j = 0ull;
    if (tree_here) {
      const uint16_t* tk = (const uint16_t*)a.tail_k;
      const uint16_t* tvv = (const uint16_t*)a.tail_v;
      const uint16_t* ktr = (const uint16_t*)a.k_tree;
      const uint16_t* vtr = (const uint16_t*)a.v_tree;
#pragma unroll
      for (int x = 0; x < TPER; ++x) {
        const int p = tid + x * NT;
        const int e = p >> 4, col = p & 15;  // entry e, channels 8col .. 8col+7
        const uint16_t* src_k;
        const uint16_t* src_v;
        if (e < rr) {
          const size_t o = (bg * (C0 - 1) + e) * kDH + col * 8;
          src_k = tk + o;
          src_v = tvv + o;
        } else {
          const int j = e < ne ? e - rr : 0;
          const size_t o = (((size_t)b * a.D + j) * a.Hkv + g) * kDH + col * 8;
          src_k = ktr + o;
          src_v = vtr + o;
        }
        if (kTFull || p < TT * 256) {
          tkp[x] = *(const uint4*)src_k;
          tvp[x] = *(const uint4*)src_v;
        }
      }
      if (tid < a.D) {
        anc_j = a.anc[(size_t)b * a.anc_ld + tid];
      }
    }

    {
      const int pid0 = load_pid(c_lo), pid1 = load_pid(c_lo + 1);
      pid_next = load_pid(c_lo + 2);
      load_chunk(c_lo, pid0, kpa, vpa);
      load_chunk(c_lo + 1, pid1, kpb, vpb);
    }

    if (tree_here) {
      __syncthreads();  // every wave is done with the LDS of the previous unit
#pragma unroll
      for (int x = 0; x < TPER; ++x) {
        const int p = tid + x * NT;
        if (kTFull || p < TT * 256) {
          const int e = p >> 4, col = p & 15;
          const uint32_t ok = e < ne ? 0xffffffffu : 0u;
          uint4 kv = tkp[x], vv = tvp[x];
          kv.x &= ok; kv.y &= ok; kv.z &= ok; kv.w &= ok;
          vv.x &= ok; vv.y &= ok; vv.z &= ok; vv.w &= ok;
          *(uint4*)(Ks + e * kKStr + col * 16) = kv;
          *(uint4*)(Vr + e * kKStr + col * 16) = vv;
        }
      }
      if (tid < a.D) {
        anc_s[tid] = anc_j & node_mask(a.D);
      }
      __syncthreads();
      if (wave_has_rows) {
        const uint64_t chain = row < a.R ? anc_s[node] : 0ull;
        const uint64_t vis = (rr > 0 ? (1ull << rr) - 1ull : 0ull) | (rr < 64 ? chain << rr : 0ull);
        f32x4 sacc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kop = *(const bf16x8*)(Ks + (16 * t + n16) * kKStr + (32 * ks + 8 * grp) * 2);
            sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[ks], sacc[t], 0, 0, 0);
          }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!((vis >> (16 * t + 4 * grp + i)) & 1ull)) sacc[t][i] = -INFINITY;  // selection
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[t][i]);
        mx = max_xor16_32(mx);
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sacc[t][i] = __builtin_amdgcn_exp2f(fmaf(sacc[t][i], a.scale_log2, -m_use));
            l_run += sacc[t][i];
          }
        // entries some row of this wave sees (wave-uniform)
        uint32_t any_lo = (uint32_t)vis, any_hi = (uint32_t)(vis >> 32);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          any_lo |= (uint32_t)__shfl_xor((int)any_lo, off, 64);
          any_hi |= (uint32_t)__shfl_xor((int)any_hi, off, 64);
        }
        const uint64_t any = ((uint64_t)any_hi << 32) | any_lo;
        // (vis, hence any, has no bit at or past ne); entry e = 16t + 4gp + i, whose
        // probability for this lane's row is held by lane (n16, gp) in sacc[t][i]
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int gp = 0; gp < 4; ++gp)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 16 * t + 4 * gp + i;
          if (!((any >> e) & 1ull)) continue;
          const float pe = __shfl(sacc[t][i], n16 + 16 * gp, 64);
          if ((vis >> e) & 1ull) {
            const char* vrow = Vr + e * kKStr;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
              const uint2 v4 = *(const uint2*)(vrow + (16 * dt + 4 * grp) * 2);
              oacc[dt][0] = fmaf(pe, bf16_bits_to_f32(v4.x & 0xffffu), oacc[dt][0]);
              oacc[dt][1] = fmaf(pe, bf16_bits_to_f32(v4.x >> 16), oacc[dt][1]);
              oacc[dt][2] = fmaf(pe, bf16_bits_to_f32(v4.y & 0xffffu), oacc[dt][2]);
              oacc[dt][3] = fmaf(pe, bf16_bits_to_f32(v4.y >> 16), oacc[dt][3]);
            }
          }
        }
      }
    }

    __syncthreads();  // every wave is done with the tree chunk's LDS and the previous unit's
    for (int c = c_lo; c < c_hi; c += 2) {
      step(c, kpa, vpa, 0);
      step(c + 1, kpb, vpb, 1);
    }

    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (row < a.R) {
      if (a.fused_tree && whole_unit) {
        // the only workgroup of this unit: normalise and write the output rows
        uint16_t* out = (uint16_t*)a.out;
        const size_t obase = (((size_t)b * a.D + node) * a.Hq + head) * kDH;
        if (live) {
          const float inv = 1.0f / l_run;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16_bits(oacc[dt][0] * inv) | ((uint32_t)f32_to_bf16_bits(oacc[dt][1] * inv) << 16);
            pk.y = (uint32_t)f32_to_bf16_bits(oacc[dt][2] * inv) | ((uint32_t)f32_to_bf16_bits(oacc[dt][3] * inv) << 16);
            *(uint2*)(out + obase + 16 * dt + 4 * grp) = pk;
          }
          if (a.lse != nullptr && grp == 0)
            a.lse[((size_t)b * a.D + node) * a.Hq + head] = (m_run + log2f(l_run)) * kLn2;
        } else {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) *(uint2*)(out + obase + 16 * dt + 4 * grp) = make_uint2(0u, 0u);
          if (a.lse != nullptr && grp == 0) a.lse[((size_t)b * a.D + node) * a.Hq + head] = -INFINITY;
        }
      } else {
        const size_t wrow = partial_row(a, part, u, w * 16 + n16);
        float* o = a.ws_o + wrow * kDH;
        if (a.nt_partials) {  // long slices: stream the partials past the caches (uniform)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) __builtin_nontemporal_store(oacc[dt], (f32x4*)(o + 16 * dt + 4 * grp));
          if (grp == 0) __builtin_nontemporal_store(f32x2{m_run, l_run}, (f32x2*)(a.ws_ml + wrow));
        } else {
          // (keeps the compiler from merging the two branches' stores into one without the hint)
          asm volatile("" ::: "memory");
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) *(f32x4*)(o + 16 * dt + 4 * grp) = oacc[dt];
          if (grp == 0) a.ws_ml[wrow] = make_float2(m_run, l_run);
          asm volatile("" ::: "memory");
        }
      }
    }
    cg = u * a.tmax + c_last;
  }
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  // NW waves per workgroup (4 for 64-row units, 8 for 128-row units): all of them load
  // (32 KB per chunk), waves whose 16 rows are all past the G*D query rows skip the
  // arithmetic.  One workgroup per slice.
  if (a.parts == 0) return hipSuccess;
  const int tt = a.fused_tree ? a.tree_tiles : 1;
  const bool paged = a.pt[0] != nullptr;  // every level or none
  const dim3 grid(a.parts + a.fold_scratch);
  if (a.unit_rows == 128) {  // 8 waves, one workgroup per CU (no folded scratch workgroups)
    if (paged) {
      if (tt == 1) hipLaunchKernelGGL((k_attn_mfma<8, 1, true>), grid, dim3(512), 0, s, a);
      else if (tt == 2) hipLaunchKernelGGL((k_attn_mfma<8, 2, true>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((k_attn_mfma<8, 4, true>), grid, dim3(512), 0, s, a);
    } else {
      if (tt == 1) hipLaunchKernelGGL((k_attn_mfma<8, 1, false>), grid, dim3(512), 0, s, a);
      else if (tt == 2) hipLaunchKernelGGL((k_attn_mfma<8, 2, false>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((k_attn_mfma<8, 4, false>), grid, dim3(512), 0, s, a);
    }
  } else if (paged) {
    if (tt == 1) hipLaunchKernelGGL((k_attn_mfma<4, 1, true>), grid, dim3(256), 0, s, a);
    else if (tt == 2) hipLaunchKernelGGL((k_attn_mfma<4, 2, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn_mfma<4, 4, true>), grid, dim3(256), 0, s, a);
  } else {
    if (tt == 1) hipLaunchKernelGGL((k_attn_mfma<4, 1, false>), grid, dim3(256), 0, s, a);
    else if (tt == 2) hipLaunchKernelGGL((k_attn_mfma<4, 2, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn_mfma<4, 4, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tv
