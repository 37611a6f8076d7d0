// Accepted-path refresh of the persistent compressed state.
// TSD-V4 §3.2 (token history, cache and compressed states must describe one
// prefix), §4.2 (only the accepted path's scratch states update the persistent
// state; rejected branches are not carried over) and §4.3 (C4 / C128 states and
// their compression-intermediate buffers).
//
// One workgroup per sequence, one thread per (KV head, channel) up to 1024; the
// accepted path is staged in LDS and checked once, and so are the pages the commits
// write (paged pools: a missing page leaves the sequence unchanged, TV_SEQ_BAD_PAGE).  Every committed element is a bit
// copy: scratch
// entries of the path nodes that close a block go to the next pool slots, the
// path leaf's open-block sums replace the open sums, path tokens extend the raw
// tail.  Counters (P, n) are written after a barrier, once every thread of the
// sequence has read the old values.  Rejected nodes are never read.
#include "accept_path.h"
#include "tv_launch.h"

namespace tv {

// The refresh of sequence b once its accepted path is in LDS (pth[0..m], m < D checked
// by the caller's path validation into path_bad) and every thread has read the old
// counters: P is sequence b's committed length before the refresh.
template <typename T>
__device__ __forceinline__ void refresh_body(int b, int D, const tv_state& st, const tv_scratch& sc,
                                             const T* __restrict__ k_tree, const T* __restrict__ v_tree, int m,
                                             int P, const int* pth, bool path_bad, int32_t* __restrict__ commit_log,
                                             int32_t* __restrict__ seq_err) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int L = st.n_levels;
  const int Hkv = st.Hkv, d = st.d, HD = Hkv * d;
  if (m >= D || P < 0 || path_bad) {
    if (tid == 0) seq_err[b] = TV_SEQ_BAD_PATH;
    return;
  }
  const int P2 = P + m + 1;
  bool full = false;
  for (int l = 0; l < L; ++l) full |= (P2 / st.lvl[l].C) > st.lvl[l].cap;
  if (full) {
    if (tid == 0) seq_err[b] = TV_SEQ_POOL_FULL;
    return;
  }
  // every page the commits write must exist (paged pools), else nothing changes
  bool page_bad = false;
  for (int l = 0; l < L; ++l)
    for (int j = P / st.lvl[l].C; j < P2 / st.lvl[l].C; ++j) {
      int page;
      page_bad |= !tile_page(st.lvl[l], b, j >> 6, &page);
    }
  if (page_bad) {
    if (tid == 0) seq_err[b] = TV_SEQ_BAD_PAGE;
    return;
  }
  const int leaf = pth[m];
  for (int l = 0; l < L; ++l) {
    const int C = st.lvl[l].C;
    T* pk = (T*)st.lvl[l].k;
    T* pvt = (T*)st.lvl[l].vt;
    const T* ek = (const T*)sc.entry_k[l];
    const T* ev = (const T*)sc.entry_v[l];
    const int j0 = P / C, j1 = P2 / C;
    for (int j = j0; j < j1; ++j) {
      const int u = pth[j * C + C - 1 - P];  // path node at the block's last position
      int page;
      tile_page(st.lvl[l], b, j >> 6, &page);  // checked above
      for (int e = tid; e < HD; e += nt) {
        const int g = e / d, dd = e - g * d;
        const size_t src = (((size_t)b * D + u) * Hkv + g) * d + dd;
        const size_t tb = tile_offset(st.lvl[l].page_table != nullptr, page, st.lvl[l].cap, st.B, Hkv, d, b, g, j >> 6);
        pk[tb + (size_t)(j & 63) * d + dd] = ek[src];
        pvt[tb + (size_t)dd * 64 + (j & 63)] = ev[src];
      }
      if (commit_log != nullptr && tid == 0) {
        int32_t* row = commit_log + (((size_t)b * L + l) * D + (j - j0)) * 2;
        row[0] = j;
        row[1] = u;
      }
    }
    const float* sok = sc.open_k[l] + ((size_t)b * D + leaf) * HD;
    const float* sov = sc.open_v[l] + ((size_t)b * D + leaf) * HD;
    for (int e = tid; e < HD; e += nt) {
      st.lvl[l].open_k[(size_t)b * HD + e] = sok[e];
      st.lvl[l].open_v[(size_t)b * HD + e] = sov[e];
    }
  }
  if (L > 0 && st.lvl[0].C > 1) {
    const int C0 = st.lvl[0].C;
    const int t_new = (P2 / C0) * C0;
    T* tk = (T*)st.tail_k;
    T* tv_ = (T*)st.tail_v;
    // positions below P keep their slot when no block closed (t_new == old start);
    // when one closed, t_new > P and only path tokens remain
    for (int pos = max(t_new, P); pos < P2; ++pos) {
      const int u = pth[pos - P];
      for (int e = tid; e < HD; e += nt) {
        const int g = e / d, dd = e - g * d;
        const size_t src = (((size_t)b * D + u) * Hkv + g) * d + dd;
        const size_t dst = (((size_t)b * Hkv + g) * (C0 - 1) + (pos - t_new)) * d + dd;
        tk[dst] = k_tree[src];
        tv_[dst] = v_tree[src];
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    st.P[b] = P2;
    for (int l = 0; l < L; ++l) st.lvl[l].n[b] = P2 / st.lvl[l].C;
  }
}

template <typename T>
__global__ __launch_bounds__(1024) void k_refresh(int D, tv_state st, tv_scratch sc,
                                                  const T* __restrict__ k_tree,
                                                  const T* __restrict__ v_tree,
                                                  const int32_t* __restrict__ m_in,
                                                  const int32_t* __restrict__ path,
                                                  int32_t* __restrict__ commit_log,
                                                  int32_t* __restrict__ seq_err) {
  __shared__ int pth[TV_MAX_D];
  __shared__ int path_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int L = st.n_levels;
  if (commit_log != nullptr)
    for (int e = tid; e < L * D * 2; e += nt) commit_log[(size_t)b * L * D * 2 + e] = -1;
  const int err = seq_err[b];
  const int m = m_in[b];
  const int P = st.P[b];
  if (tid == 0) path_bad = 0;
  __syncthreads();  // log prefill and the reads above happen before any later write
  if (err != TV_SEQ_OK || m < 0) return;
  if (tid < D) {
    const int v = path[(size_t)b * D + tid];
    pth[tid] = v;
    if (tid <= m && (v < 0 || v >= D)) atomicOr(&path_bad, 1);
  }
  __syncthreads();
  refresh_body<T>(b, D, st, sc, k_tree, v_tree, m, P, pth, path_bad != 0, commit_log, seq_err);
}

// Acceptance and refresh in one launch (one workgroup per sequence): the first wave
// selects the accepted path into LDS (and writes m, path and bonus as tv_accept does),
// then the workgroup refreshes from it.  Saves a launch and the round trip that reads m
// and the path back; results are those of tv_accept followed by tv_refresh_state.
template <typename T>
__global__ __launch_bounds__(1024) void k_accept_refresh(int D, tv_state st, tv_scratch sc,
                                                         const int32_t* __restrict__ parents,
                                                         const uint64_t* __restrict__ anc,
                                                         const int32_t* __restrict__ depth,
                                                         const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ target,
                                                         const T* __restrict__ k_tree,
                                                         const T* __restrict__ v_tree,
                                                         int32_t* __restrict__ m_out, int32_t* __restrict__ path,
                                                         int32_t* __restrict__ bonus,
                                                         int32_t* __restrict__ commit_log,
                                                         int32_t* __restrict__ seq_err) {
  __shared__ int pth[TV_MAX_D];
  __shared__ int m_s;
  __shared__ int path_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int L = st.n_levels;
  if (commit_log != nullptr)
    for (int e = tid; e < L * D * 2; e += nt) commit_log[(size_t)b * L * D * 2 + e] = -1;
  const int err = seq_err[b];
  const int P = st.P[b];
  if (tid < 64) {  // the first wave: every path slot -1, then the accepted path
    if (tid < D) pth[tid] = -1;
    const int m = accept_one(b, D, parents, anc, depth, draft, target, err, m_out, path, bonus, pth);
    if (tid == 0) {
      m_s = m;
      path_bad = 0;
    }
  }
  __syncthreads();  // the path is in LDS; the log prefill and the reads above are done
  const int m = m_s;
  if (err != TV_SEQ_OK || m < 0) return;
  // slots 0..m hold one node each for a plan from tv_build_tree_mask; checked as
  // tv_refresh_state checks a path it is given
  if (tid < D && tid <= m && (pth[tid] < 0 || pth[tid] >= D)) atomicOr(&path_bad, 1);
  __syncthreads();
  refresh_body<T>(b, D, st, sc, k_tree, v_tree, m, P, pth, path_bad != 0, commit_log, seq_err);
}

hipError_t launch_accept_refresh(int D, const tv_state& st, const tv_scratch& sc, const int32_t* parents,
                                 const uint64_t* anc, const int32_t* depth, const int32_t* draft,
                                 const int32_t* target, const void* k_tree, const void* v_tree, int32_t* m,
                                 int32_t* path, int32_t* bonus, int32_t* commit_log, int32_t* seq_err,
                                 hipStream_t s) {
  if (st.B == 0) return hipSuccess;
  dim3 grid(st.B), block(st.Hkv * st.d >= 1024 ? 1024 : ((st.Hkv * st.d + 63) / 64) * 64);
  if (st.dtype == TV_BF16)
    hipLaunchKernelGGL(k_accept_refresh<uint16_t>, grid, block, 0, s, D, st, sc, parents, anc, depth, draft,
                       target, (const uint16_t*)k_tree, (const uint16_t*)v_tree, m, path, bonus, commit_log,
                       seq_err);
  else
    hipLaunchKernelGGL(k_accept_refresh<float>, grid, block, 0, s, D, st, sc, parents, anc, depth, draft, target,
                       (const float*)k_tree, (const float*)v_tree, m, path, bonus, commit_log, seq_err);
  return hipGetLastError();
}

hipError_t launch_refresh(int D, const tv_state& st, const tv_scratch& sc, const void* k_tree,
                          const void* v_tree, const int32_t* m, const int32_t* path,
                          int32_t* commit_log, int32_t* seq_err, hipStream_t s) {
  if (st.B == 0) return hipSuccess;
  dim3 grid(st.B), block(st.Hkv * st.d >= 1024 ? 1024 : ((st.Hkv * st.d + 63) / 64) * 64);
  if (st.dtype == TV_BF16)
    hipLaunchKernelGGL(k_refresh<uint16_t>, grid, block, 0, s, D, st, sc, (const uint16_t*)k_tree,
                       (const uint16_t*)v_tree, m, path, commit_log, seq_err);
  else
    hipLaunchKernelGGL(k_refresh<float>, grid, block, 0, s, D, st, sc, (const float*)k_tree,
                       (const float*)v_tree, m, path, commit_log, seq_err);
  return hipGetLastError();
}

}  // namespace tv
