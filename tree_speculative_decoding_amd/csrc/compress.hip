// Compressed state of a raw committed prefix.  TSD-V4 §2.2: CSA/HCA build
// compressed representations along the sequence axis at several granularities;
// the compressor itself is not given there, the stand-in is the unweighted mean
// of every complete aligned block of C positions (per level, per KV head, K and V
// separately), with an fp32 running sum for the incomplete last block.
//
// k_compress_entries: one thread per (entry, channel), channels fastest so the
//   raw reads of a block are coalesced; sums in fp32 in position order.
// k_compress_finish: one workgroup per (sequence, KV head): open-block sums, the
//   finest level's raw tail, counts and the per-sequence status (a paged pool whose
//   page table lacks a page the entries need flags the sequence TV_SEQ_BAD_PAGE).
#include "tv_launch.h"

namespace tv {

__device__ __forceinline__ bool prefix_ok(const tv_state& st, int P, int max_len, int* code) {
  if (P < 0 || P > max_len) {
    *code = TV_SEQ_BAD_PREFIX;
    return false;
  }
  for (int l = 0; l < st.n_levels; ++l)
    if (P / st.lvl[l].C > st.lvl[l].cap) {
      *code = TV_SEQ_POOL_FULL;
      return false;
    }
  *code = TV_SEQ_OK;
  return true;
}

template <typename T>
__global__ __launch_bounds__(256) void k_compress_entries(tv_state st, int l, const T* __restrict__ raw_k,
                                                          const T* __restrict__ raw_v, int max_len) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int d = st.d;
  const int P = st.P[b];
  int code;
  if (!prefix_ok(st, P, max_len, &code)) return;
  const int C = st.lvl[l].C;
  const long item = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int j = (int)(item / d), dd = (int)(item % d);
  if (j >= P / C) return;
  const size_t rbase = ((size_t)b * st.Hkv + g) * max_len;
  float sk = 0.f, sv = 0.f;
  for (int t = 0; t < C; ++t) {
    const size_t o = (rbase + (size_t)j * C + t) * d + dd;
    sk += Elem<T>::load(raw_k, o);
    sv += Elem<T>::load(raw_v, o);
  }
  int page;
  if (!tile_page(st.lvl[l], b, j >> 6, &page)) return;  // flagged by k_compress_finish
  const size_t tb = tile_offset(st.lvl[l].page_table != nullptr, page, st.lvl[l].cap, st.B, st.Hkv, d, b, g, j >> 6);
  Elem<T>::store((T*)st.lvl[l].k, tb + (size_t)(j & 63) * d + dd, sk / (float)C);
  Elem<T>::store((T*)st.lvl[l].vt, tb + (size_t)dd * 64 + (j & 63), sv / (float)C);
}

template <typename T>
__global__ __launch_bounds__(256) void k_compress_finish(tv_state st, const T* __restrict__ raw_k,
                                                         const T* __restrict__ raw_v, int max_len,
                                                         int32_t* __restrict__ seq_err) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int d = st.d, Hkv = st.Hkv;
  const int P = st.P[b];
  int code;
  bool ok = prefix_ok(st, P, max_len, &code);
  // every page the entries went to must exist (paged pools)
  for (int l = 0; ok && l < st.n_levels; ++l)
    for (int t = 0; t * 64 < P / st.lvl[l].C; ++t) {
      int page;
      if (!tile_page(st.lvl[l], b, t, &page)) {
        ok = false;
        code = TV_SEQ_BAD_PAGE;
        break;
      }
    }
  if (g == 0 && threadIdx.x == 0) seq_err[b] = code;
  if (!ok) return;
  const size_t rbase = ((size_t)b * Hkv + g) * max_len;
  for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
    for (int l = 0; l < st.n_levels; ++l) {
      const int C = st.lvl[l].C;
      float sk = 0.f, sv = 0.f;
      for (int t = (P / C) * C; t < P; ++t) {
        sk += Elem<T>::load(raw_k, (rbase + t) * d + dd);
        sv += Elem<T>::load(raw_v, (rbase + t) * d + dd);
      }
      st.lvl[l].open_k[((size_t)b * Hkv + g) * d + dd] = sk;
      st.lvl[l].open_v[((size_t)b * Hkv + g) * d + dd] = sv;
    }
    if (st.n_levels > 0 && st.lvl[0].C > 1) {
      const int C0 = st.lvl[0].C;
      const int t0 = (P / C0) * C0;
      for (int t = t0; t < P; ++t) {
        const size_t dst = (((size_t)b * Hkv + g) * (C0 - 1) + (t - t0)) * d + dd;
        ((T*)st.tail_k)[dst] = raw_k[(rbase + t) * d + dd];
        ((T*)st.tail_v)[dst] = raw_v[(rbase + t) * d + dd];
      }
    }
  }
  if (g == 0 && threadIdx.x == 0)
    for (int l = 0; l < st.n_levels; ++l) st.lvl[l].n[b] = P / st.lvl[l].C;
}

template <typename T>
static hipError_t launch_compress_t(const tv_state& st, const T* rk, const T* rv, int max_len,
                                    int32_t* seq_err, hipStream_t s) {
  for (int l = 0; l < st.n_levels; ++l) {
    const long max_entries = max_len / st.lvl[l].C;
    if (max_entries == 0) continue;
    const long items = max_entries * st.d;
    dim3 grid((unsigned)((items + 255) / 256), st.Hkv, st.B);
    hipLaunchKernelGGL(k_compress_entries<T>, grid, dim3(256), 0, s, st, l, rk, rv, max_len);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_compress_finish<T>, dim3(st.Hkv, st.B), dim3(st.d), 0, s, st, rk, rv, max_len,
                     seq_err);
  return hipGetLastError();
}

hipError_t launch_compress(const tv_state& st, const void* raw_k, const void* raw_v, int max_len,
                           int32_t* seq_err, hipStream_t s) {
  if (st.B == 0) return hipSuccess;
  if (st.dtype == TV_BF16)
    return launch_compress_t(st, (const uint16_t*)raw_k, (const uint16_t*)raw_v, max_len, seq_err, s);
  return launch_compress_t(st, (const float*)raw_k, (const float*)raw_v, max_len, seq_err, s);
}

}  // namespace tv
