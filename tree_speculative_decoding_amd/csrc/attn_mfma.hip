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
//      then written to LDS (straight copies, padded rows);
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
constexpr int kPieces = 2 * kChunk * kDH * 2 / 16;  // 16-byte pieces per chunk (K + V^T)
}  // namespace

template <int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_mfma(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int PER = (kPieces + NT - 1) / NT;
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

  uint4 pre[PER];
  // piece p < 1024: K row p/16, 16-byte column p%16; p >= 1024: V^T row (p-1024)/8, column %8
  auto load_chunk = [&](int c) {
    int lvl, e0, cnt;
    chunk_entries(n0, T0, n1, c, &lvl, &e0, &cnt);
    const char* pk = (const char*)a.pk[lvl];
    const char* pv = (const char*)a.pvt[lvl];
    const size_t cap = (size_t)a.cap[lvl];
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int p = tid + x * NT;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (p < 1024) {
        const int r = p >> 4, col = p & 15;
        if (r < cnt) v = *(const uint4*)(pk + ((bg * cap + e0 + r) * kDH + col * 8) * 2);
      } else if (p < kPieces) {
        const int q = p - 1024;
        const int dr = q >> 3, col = q & 7;
        const int e_first = col * 8;
        if (e_first < cnt) {
          v = *(const uint4*)(pv + ((bg * kDH + dr) * cap + e0 + e_first) * 2);
          const int keep = cnt - e_first;  // entries of this piece that are committed
          if (keep < 8) {
            // zero uncommitted entries (select, never arithmetic: they may hold anything)
            uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              const uint32_t lo_ok = (2 * h) < keep ? 0x0000ffffu : 0u;
              const uint32_t hi_ok = (2 * h + 1) < keep ? 0xffff0000u : 0u;
              w4[h] &= (lo_ok | hi_ok);
            }
            v = make_uint4(w4[0], w4[1], w4[2], w4[3]);
          }
        }
      }
      pre[x] = v;
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int p = tid + x * NT;
      if (p < 1024) {
        *(uint4*)(Ks + (p >> 4) * kKStr + (p & 15) * 16) = pre[x];
      } else if (p < kPieces) {
        const int q = p - 1024;
        *(uint4*)(Vs + (q >> 3) * kVStr + (q & 7) * 16) = pre[x];
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
    store_chunk();
    __syncthreads();
    if (c + 1 < c_hi) load_chunk(c + 1);  // in flight while this chunk is computed

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
  // waves per workgroup: enough 16-row tiles for the rows of one 64-row block
  const int rows = a.row_blocks > 1 ? 64 : a.R;
  const int nw = (rows + 15) / 16;
  dim3 grid(a.splits, a.Hkv * a.row_blocks, a.B);
  switch (nw) {
    case 1: hipLaunchKernelGGL(k_attn_mfma<1>, grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_attn_mfma<2>, grid, dim3(128), 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_attn_mfma<3>, grid, dim3(192), 0, s, a); break;
    default: hipLaunchKernelGGL(k_attn_mfma<4>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace tv
