// Branch-aware verify attention, shared-prefix stream: bf16 MFMA kernel (gfx950).
// TSD-V4 §3.1 (each candidate attends to the accepted context; the tree part is
// added by the merge kernel), §2.2 (the context is the multi-resolution
// compressed history), §2.1 / §5.3 (verification of many candidates is
// memory-bound at small batch: the prefix is read once for all G*D query rows of
// a KV head).
//
// Grid (split, KV head x row block, sequence), NW waves per workgroup, 16 query
// rows per wave (rows r = node * G + head-in-group).  Per 64-entry chunk:
//   1. the K chunk (64 x 128, row-major) and the transposed V chunk (128 x 64)
//      are loaded with 16-byte coalesced loads into registers one chunk ahead,
//      all issued back to back, then written to LDS (straight copies, padded rows);
//   2. S^T = K Q^T with v_mfma_f32_16x16x32_bf16: the K chunk is the A operand
//      (16 entries x 32 channels per lane group), Q^T the B operand kept in
//      registers for the whole kernel; the accumulator gives each lane one query
//      row and 4 entries per 16-entry tile;
//   3. online softmax in base-2 units: the row max is combined across the four
//      lane groups by two xor shuffles; each lane keeps its own partial sum;
//   4. O^T += V^T P^T with the same MFMA: the transposed V chunk is the A operand
//      (16 channels x 32 entries) read from LDS in the entry order the softmax
//      lanes hold, P^T (bf16) the B operand straight from registers, and the
//      accumulator again gives each lane its own query row, so the rescale by
//      exp2(m_old - m_new) needs no data movement.
// The unnormalised output rows, running max and sum go to the workspace.
#include "tv_common.h"

namespace tv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int kDH = 128;        // head dim handled by this kernel
constexpr int kChunk = 64;      // entries per chunk
constexpr int kKStr = kDH * 2 + 16;      // LDS bytes per K row (padded)
constexpr int kVStr = kChunk * 2 + 16;   // LDS bytes per V^T row (padded)
constexpr int kLdsBytes = kChunk * kKStr + kDH * kVStr;
}  // namespace

// At most 168 VGPRs, so three workgroups fit on a CU (LDS allows four).
template <int NW>
__global__ __launch_bounds__(NW * 64, 3) void k_attn_mfma(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int PER = (1024 + NT - 1) / NT;   // K pieces (and V pieces) per thread
  constexpr bool kFull = 1024 % NT == 0;
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  char* Ks = smem;
  char* Vs = smem + kChunk * kKStr;

  const int s = blockIdx.x;
  const int g = blockIdx.y % a.Hkv;
  const int rb = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, grp = lane >> 4;
  const size_t bg = (size_t)b * a.Hkv + g;

  // Q^T operand: lane (n16, grp), k-step ks holds Q[row][32ks + 8grp .. +7]
  const int row = rb * 64 + w * 16 + n16;
  const bool wave_has_rows = rb * 64 + w * 16 < a.R;  // wave-uniform
  bf16x8 qop[4];
  {
    const uint16_t* q = (const uint16_t*)a.q;
    if (row < a.R) {
      const int i = row / a.G, hh = row - i * a.G;
      const uint16_t* qr = q + (((size_t)b * a.D + i) * a.Hq + g * a.G + hh) * kDH;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qop[ks] = *(const bf16x8*)(qr + 32 * ks + 8 * grp);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qop[ks] = bf16x8{};
    }
  }

  const bool live = a.seq_err == nullptr || a.seq_err[b] == TV_SEQ_OK;
  const int n0 = a.n_levels > 0 ? level_count(a.pn[0], b, a.cap[0]) : 0;
  const int n1 = a.n_levels > 1 ? level_count(a.pn[1], b, a.cap[1]) : 0;
  const int T0 = (n0 + 63) / 64, T1 = (n1 + 63) / 64;
  const int per = (T0 + T1 + a.splits - 1) / a.splits;
  const int c_lo = s * per;
  const int c_hi = live ? min(T0 + T1, c_lo + per) : c_lo;

  // Pieces: 1024 16-byte pieces of K (row p/16, column p%16) and 1024 of V^T (row p/8,
  // column p%8) per chunk; thread tid takes pieces tid, tid + NT, ...  A chunk is
  // 64-aligned in its pool and a pool's capacity is a multiple of 64, so all 64 entries of
  // a chunk are in bounds: every piece is loaded unconditionally (no data-dependent code
  // between the loads, so they are all in flight together) and entries past the committed
  // count are zeroed by selection when the chunk is written to LDS.
  uint4 kpre[PER], vpre[PER];
  auto load_chunk = [&](int c) {
    int lvl, e0, cnt;
    chunk_entries(n0, T0, n1, c, &lvl, &e0, &cnt);
    const uint32_t cap = (uint32_t)a.cap[lvl];
    const char* kb = (const char*)a.pk[lvl] + (bg * cap + e0) * (kDH * 2);   // uniform
    const char* vb = (const char*)a.pvt[lvl] + (bg * kDH * cap + e0) * 2;    // uniform
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int p = tid + x * NT;
      if (kFull || p < 1024) {
        kpre[x] = *(const uint4*)(kb + (uint32_t)p * 16);  // K rows are 256 B: piece p at 16p
        vpre[x] = *(const uint4*)(vb + ((uint32_t)(p >> 3) * cap + (uint32_t)(p & 7) * 8) * 2);
      }
    }
  };
  auto store_chunk = [&](int cnt) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int p = tid + x * NT;
      if (kFull || p < 1024) {
        const uint32_t krow_ok = (p >> 4) < cnt ? 0xffffffffu : 0u;
        uint4 kv = kpre[x];
        kv.x &= krow_ok; kv.y &= krow_ok; kv.z &= krow_ok; kv.w &= krow_ok;
        *(uint4*)(Ks + (p >> 4) * kKStr + (p & 15) * 16) = kv;
        const int keep = cnt - (p & 7) * 8;  // committed entries among this piece's 8
        uint4 vv = vpre[x];
        vv.x &= (keep > 0 ? 0x0000ffffu : 0u) | (keep > 1 ? 0xffff0000u : 0u);
        vv.y &= (keep > 2 ? 0x0000ffffu : 0u) | (keep > 3 ? 0xffff0000u : 0u);
        vv.z &= (keep > 4 ? 0x0000ffffu : 0u) | (keep > 5 ? 0xffff0000u : 0u);
        vv.w &= (keep > 6 ? 0x0000ffffu : 0u) | (keep > 7 ? 0xffff0000u : 0u);
        *(uint4*)(Vs + (p >> 3) * kVStr + (p & 7) * 16) = vv;
      }
    }
  };

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (c_lo < c_hi) load_chunk(c_lo);
  for (int c = c_lo; c < c_hi; ++c) {
    int lvl, e0, cnt;
    chunk_entries(n0, T0, n1, c, &lvl, &e0, &cnt);
    __syncthreads();  // every wave is done reading the previous chunk
    store_chunk(cnt);
    __syncthreads();
    if (c + 1 < c_hi) load_chunk(c + 1);  // in flight while this chunk is computed
    if (!wave_has_rows) continue;

    // S^T tiles: sacc[t] lane (n16, grp) = S[row n16][entry 16t + 4grp + i]
    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kop = *(const bf16x8*)(Ks + (16 * t + n16) * kKStr + (32 * ks + 8 * grp) * 2);
        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[ks], sacc[t], 0, 0, 0);
      }
    }
    // online softmax over this chunk
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 16 * t + 4 * grp + i;
        const float x = sacc[t][i] * a.scale_log2;
        sacc[t][i] = e < cnt ? x : -INFINITY;
        mx = fmaxf(mx, sacc[t][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);  // finite: cnt >= 1
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pop[2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sacc[t][i] - m_new);
        psum += p;
        pop[t >> 1][(t & 1) * 4 + i] = (__bf16)p;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // O^T += V^T P^T; k-step h covers entries 32h + {4grp..4grp+3} and 32h + 16 + {4grp..4grp+3}
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      oacc[dt] *= alpha;
      const char* vrow = Vs + (16 * dt + n16) * kVStr;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x4 lo = *(const bf16x4*)(vrow + (32 * h + 4 * grp) * 2);
        const bf16x4 hi = *(const bf16x4*)(vrow + (32 * h + 16 + 4 * grp) * 2);
        const bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[h], oacc[dt], 0, 0, 0);
      }
    }
  }

  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (row < a.R) {
    const size_t wrow = ((bg * a.splits + s) * a.R + row);
    float* o = a.ws_o + wrow * kDH;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *(f32x4*)(o + 16 * dt + 4 * grp) = oacc[dt];
    if (grp == 0) a.ws_ml[wrow] = make_float2(m_run, l_run);
  }
}

hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s) {
  // Always four waves: all of them load (32 KB per chunk), waves whose 16 rows are all
  // past the G*D query rows skip the arithmetic.
  dim3 grid(a.splits, a.Hkv * a.row_blocks, a.B);
  hipLaunchKernelGGL(k_attn_mfma<4>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tv
