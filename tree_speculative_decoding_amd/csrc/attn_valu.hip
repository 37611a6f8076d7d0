// Branch-aware verify attention, shared-prefix stream: fp32 vector-ALU kernel.
// TSD-V4 §3.1 (each candidate attends to the accepted context; the tree part is
// added by the merge kernel) and §2.2 (the context is the multi-resolution
// compressed history).  Used for fp32 inputs and for shapes the MFMA kernel does
// not take (bf16 with head dim 64).
//
// One persistent workgroup per slice of the units' chunks (as in the MFMA kernel);
// 256 threads = 64 query rows x 4.  The 64-entry chunks are streamed through LDS in
// 32-entry tiles (K row-major, V transposed as in HBM); each row keeps an
// online-softmax running max (base-2 units), a per-thread partial sum and a quarter
// of the output row in registers.  The partial (max, sum, unnormalised output) of
// every unit goes to the workspace for the merge kernel.
#include "tv_launch.h"

namespace tv {

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_attn_valu(AttnArgs a) {
  constexpr int TK = 32;
  constexpr int RBLK = 64;
  constexpr int DQ = DH / 4;
  __shared__ float Qs[RBLK][DH + 1];
  __shared__ float Ks[TK][DH + 1];
  __shared__ float Vs[DH][TK + 1];
  __shared__ float Ps[RBLK][TK + 1];

  const int tid = threadIdx.x;
  const int r_loc = tid >> 2, part = tid & 3;
  const T* q = (const T*)a.q;

  int cg = slice_begin(a, blockIdx.x);
  const int cend = slice_begin(a, blockIdx.x + 1);
  while (cg < cend) {
    const int u = cg / a.tmax;
    const int c_first = cg - u * a.tmax;
    const int c_last = min(a.tmax, cend - u * a.tmax);
    const int rb = u % a.row_blocks;
    const int g = (u / a.row_blocks) % a.Hkv;
    const int b = u / (a.row_blocks * a.Hkv);
    const size_t bg = (size_t)b * a.Hkv + g;
    const int row = rb * RBLK + r_loc;

    __syncthreads();  // the previous unit is done with Qs
    for (int e = tid; e < RBLK * DH; e += 256) {
      const int rr = e / DH, dd = e - rr * DH;
      const int rw = rb * RBLK + rr;
      float v = 0.f;
      if (rw < a.R) {
        const int i = rw / a.G, hh = rw - i * a.G;
        v = Elem<T>::load(q, (((size_t)b * a.D + i) * a.Hq + g * a.G + hh) * DH + dd);
      }
      Qs[rr][dd] = v;
    }

    const bool live = a.seq_err == nullptr || a.seq_err[b] == TV_SEQ_OK;
    const int n0 = a.n_levels > 0 ? level_count(a.pn[0], b, a.cap[0]) : 0;
    const int n1 = a.n_levels > 1 ? level_count(a.pn[1], b, a.cap[1]) : 0;
    const int T0 = (n0 + 63) / 64, T1 = (n1 + 63) / 64;
    const int c_lo = c_first;
    const int c_hi = live ? min(c_last, T0 + T1) : c_first;

    float o[DQ];
#pragma unroll
    for (int x = 0; x < DQ; ++x) o[x] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    for (int c = c_lo; c < c_hi; ++c) {
      int lvl, e0, cnt;
      chunk_entries(n0, T0, n1, c, &lvl, &e0, &cnt);
      const T* pk = (const T*)a.pk[lvl];
      const T* pvt = (const T*)a.pvt[lvl];
      // the chunk is one 64-entry tile: contiguous by (b, g, tile), paged by its page id
      const bool paged = a.pt[lvl] != nullptr;
      const int tile = e0 >> 6;
      const int page = paged ? a.pt[lvl][(size_t)b * a.ppseq[lvl] + tile] : 0;
      const bool page_ok = !paged || (page >= 0 && page < a.npages[lvl]);
      const size_t tb = tile_offset(paged, page, a.cap[lvl], a.B, a.Hkv, DH, b, g, tile);
      for (int sub = 0; sub * TK < cnt; ++sub) {
        const int base = e0 + sub * TK;
        const int n_sub = min(TK, cnt - sub * TK);
        __syncthreads();  // previous tile fully consumed (and Q staged on the first pass)
        for (int e = tid; e < TK * DH; e += 256) {
          const int k = e / DH, dd = e - k * DH;
          Ks[k][dd] = k < n_sub && page_ok ? Elem<T>::load(pk, tb + (size_t)((base + k) & 63) * DH + dd) : 0.f;
        }
        for (int e = tid; e < DH * TK; e += 256) {
          const int dd = e / TK, k = e - dd * TK;
          Vs[dd][k] = k < n_sub && page_ok ? Elem<T>::load(pvt, tb + (size_t)dd * 64 + ((base + k) & 63)) : 0.f;
        }
        __syncthreads();
        float sc[TK / 4];
        float tmax = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < TK / 4; ++jj) {
          const int k = part + 4 * jj;
          float acc = 0.f;
#pragma unroll 8
          for (int dd = 0; dd < DH; ++dd) acc = fmaf(Qs[r_loc][dd], Ks[k][dd], acc);
          const float x = acc * a.scale_log2;
          sc[jj] = k < n_sub ? x : -INFINITY;
          tmax = fmaxf(tmax, sc[jj]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 64));
        const float m_new = fmaxf(m_run, tmax);  // finite: n_sub >= 1
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int jj = 0; jj < TK / 4; ++jj) {
          const int k = part + 4 * jj;
          const float p = k < n_sub ? exp2f(sc[jj] - m_new) : 0.f;
          Ps[r_loc][k] = p;
          psum += p;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < DQ; ++x) {
          const int dd = part * DQ + x;
          float acc = o[x] * alpha;
#pragma unroll 8
          for (int k = 0; k < TK; ++k) acc = fmaf(Ps[r_loc][k], Vs[dd][k], acc);
          o[x] = acc;
        }
      }
    }
    l_run += __shfl_xor(l_run, 1, 64);
    l_run += __shfl_xor(l_run, 2, 64);
    if (row < a.R) {
      const size_t wr = partial_row(a, blockIdx.x, u, r_loc);
#pragma unroll
      for (int x = 0; x < DQ; ++x) a.ws_o[wr * DH + part * DQ + x] = o[x];
      if (part == 0) a.ws_ml[wr] = make_float2(m_run, l_run);
    }
    cg = u * a.tmax + c_last;
  }
}

hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t s) {
  if (a.parts == 0) return hipSuccess;
  if (a.unit_rows != 64) return hipErrorInvalidValue;  // this kernel's units are 64 rows
  dim3 grid(a.parts), block(256);
  if (a.dtype == TV_BF16) {
    if (a.d == 128)
      hipLaunchKernelGGL((k_attn_valu<uint16_t, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_valu<uint16_t, 64>), grid, block, 0, s, a);
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL((k_attn_valu<float, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_valu<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tv
