// Accepted-path refresh of the persistent compressed state.
// TSD-V4 §3.2 (token history, cache and compressed states must describe one
// prefix), §4.2 (only the accepted path's scratch states update the persistent
// state; rejected branches are not carried over) and §4.3 (C4 / C128 states and
// their compression-intermediate buffers).
//
// One workgroup per sequence, one thread per (KV head, channel) up to 1024; the
// accepted path is staged in LDS and checked once, and so are the pages the commits
// write (paged pools: a missing page leaves the sequence unchanged, TV_SEQ_BAD_PAGE).
// Every committed element is a bit copy: scratch entries of the path nodes that close a
// block go to the next pool slots (except those the verify already wrote there: nodes of
// the scratch pad's in-place chain, TSD-V4 §4.3's refresh skip), the path leaf's
// open-block sums replace the open sums, path tokens extend the raw tail.  A level marked
// in scratch.deferred (TSD-V4 §4.3: the coarse level's writes delayed and combined once the
// accepted path is known) has no scratch states: its open sum and the entries the path
// closes are computed here from the committed open sum and the path tokens, in path
// order in fp32 with one rounding per entry -- the additions the scratch pad would have
// made along the same chain, so the results are the same bits.  Counters (P,
// n) are written after a barrier, once every thread of the sequence has read the old
// values.  Rejected nodes are never read.
#include "accept_path.h"
#include "tv_launch.h"

namespace tv {

// LDS of a refresh workgroup: the accepted path, the blocks it commits and the
// validation flags (bit 0: a path node out of range, bit 1: a page missing).
struct RefreshLds {
  static constexpr int kMaxCommits = 2 * (TV_MAX_D + 1);  // per level at most (m + 1)/C + 1
  int pth[TV_MAX_D];
  int it_l[kMaxCommits], it_j[kMaxCommits], it_u[kMaxCommits];
  // element offset of the block's tile for KV head 0, and from one head's tile to the
  // next (tile_offset is linear in the head in every pool layout)
  size_t it_tile0[kMaxCommits], it_gstep[kMaxCommits];
  int cp[kMaxCommits];  // the listed commits to copy (those not already in place), any order
  int ncp;
  int bad;
};

// A storage element's bits, widened to 32 (so that no two elements share a register).
template <typename T>
struct Bits;
template <>
struct Bits<uint16_t> {
  static __device__ __forceinline__ uint32_t ld(const uint16_t* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void st(uint16_t* p, size_t i, uint32_t v) { p[i] = (uint16_t)v; }
};
template <>
struct Bits<float> {
  static __device__ __forceinline__ uint32_t ld(const float* p, size_t i) { return __float_as_uint(p[i]); }
  static __device__ __forceinline__ void st(float* p, size_t i, uint32_t v) { p[i] = __uint_as_float(v); }
};

// A storage element's bits widened to fp32, and an fp32 value rounded once (to nearest
// even) to a storage element's bits.
template <typename T>
struct Wide;
template <>
struct Wide<uint16_t> {
  static __device__ __forceinline__ float f(uint32_t v) { return bf16_bits_to_f32(v); }
  static __device__ __forceinline__ uint32_t bits(float x) { return f32_to_bf16_bits(x); }
};
template <>
struct Wide<float> {
  static __device__ __forceinline__ float f(uint32_t v) { return __uint_as_float(v); }
  static __device__ __forceinline__ uint32_t bits(float x) { return __float_as_uint(x); }
};

// Commits and tail tokens whose loads are issued together, ahead of any store (the
// common trees need one batch of each; longer accepted paths take more).
constexpr int kCommitBatch = 8;
constexpr int kTailBatch = 4;

// The refresh of sequence b: sh.pth[0..m] holds the accepted path and sh.bad is 0 (both
// behind a barrier), and every thread has read the old counters: P is the sequence's
// committed length before the refresh.  The threads first list the blocks the path
// closes (one thread per block: its level, slot, closing node and page), checking the
// path and the pages; then each thread copies its channels of every listed entry, the
// leaf's open sums and the new tail tokens, with all of a batch's loads issued before its
// stores (the sources, scratch pad and tree tokens, are never written here).
// `in_place` is the mask of nodes whose entries the verify wrote into the pools (0: none).
template <typename T>
__device__ __forceinline__ void refresh_body(int b, int D, const tv_state& st, const tv_scratch& sc,
                                             const T* __restrict__ k_tree, const T* __restrict__ v_tree, int m,
                                             int P, uint64_t in_place, RefreshLds& sh,
                                             int32_t* __restrict__ commit_log, int32_t* __restrict__ seq_err) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int L = st.n_levels;
  const int Hkv = st.Hkv, d = st.d, HD = Hkv * d;
  if (m >= D || P < 0) {  // uniform
    if (tid == 0) seq_err[b] = TV_SEQ_BAD_PATH;
    return;
  }
  const int P2 = P + m + 1;
  bool full = false;
  int j0[2] = {0, 0}, nc[2] = {0, 0};
  for (int l = 0; l < L; ++l) {
    full |= (P2 / st.lvl[l].C) > st.lvl[l].cap;
    j0[l] = P / st.lvl[l].C;
    nc[l] = P2 / st.lvl[l].C - j0[l];
  }
  const int ncom = nc[0] + nc[1];
  if (tid <= m && (sh.pth[tid] < 0 || sh.pth[tid] >= D)) atomicOr(&sh.bad, 1);  // (m < D <= threads)
  // (up to 2 (D + 1) blocks, more than the threads of a small workgroup)
  for (int i = full ? ncom : tid; i < ncom; i += nt) {
    const bool l1 = i >= nc[0];  // levels are picked by selection, not by a run-time index
    const tv_level& lv = l1 ? st.lvl[1] : st.lvl[0];
    const int C = lv.C;
    const int j = l1 ? j0[1] + i - nc[0] : j0[0] + i;
    int page;
    if (!tile_page(lv, b, j >> 6, &page)) atomicOr(&sh.bad, 2);
    const bool paged = lv.page_table != nullptr;
    const size_t t0 = tile_offset(paged, page, lv.cap, st.B, Hkv, d, b, 0, j >> 6);
    sh.it_l[i] = l1 ? 1 : 0;
    sh.it_j[i] = j;
    const int u = sh.pth[j * C + C - 1 - P];  // path node at the block's last position
    sh.it_u[i] = u;
    // not yet in its slot (a deferred level's entries are computed below, not copied)
    if (!((sc.deferred >> (l1 ? 1 : 0)) & 1u) && (!((in_place >> (u & 63)) & 1ull) || u < 0))
      sh.cp[atomicAdd(&sh.ncp, 1)] = i;
    sh.it_tile0[i] = t0;
    sh.it_gstep[i] = tile_offset(paged, page, lv.cap, st.B, Hkv, d, b, 1, j >> 6) - t0;
  }
  __syncthreads();
  const int bad = sh.bad;
  const int ncp = sh.ncp;
  if (bad != 0 || full) {  // uniform; the state is left unchanged
    if (tid == 0) seq_err[b] = (bad & 1) ? TV_SEQ_BAD_PATH : full ? TV_SEQ_POOL_FULL : TV_SEQ_BAD_PAGE;
    return;
  }
  if (commit_log != nullptr)
    for (int i = tid; i < ncom; i += nt) {
      const int l = sh.it_l[i];
      int32_t* row = commit_log + (((size_t)b * L + l) * D + (sh.it_j[i] - (l ? j0[1] : j0[0]))) * 2;
      row[0] = sh.it_j[i];
      row[1] = sh.it_u[i];
    }
  const int leaf = sh.pth[m];
  const bool def0 = L > 0 && (sc.deferred & 1u), def1 = L > 1 && (sc.deferred & 2u);
  // the finest level's raw tail: positions [t0, P2) come from the path; positions below
  // P keep their slot when no block closed (t_new == old start), when one closed t_new > P
  // and only path tokens remain
  const int C0 = L > 0 ? st.lvl[0].C : 1;
  const int t_new = C0 > 1 ? (P2 / C0) * C0 : P2;
  const int t0 = max(t_new, P);
  const int ntail = C0 > 1 ? P2 - t0 : 0;
  const T* ek0 = (const T*)sc.entry_k[0];
  const T* ek1 = (const T*)sc.entry_k[1];
  const T* ev0 = (const T*)sc.entry_v[0];
  const T* ev1 = (const T*)sc.entry_v[1];
  T* tail_k = (T*)st.tail_k;
  T* tail_v = (T*)st.tail_v;
  for (int e = tid; e < HD; e += nt) {
    const int g = e / d, dd = e - g * d;
    const size_t seq_rows = (size_t)b * D;
    // loads: the leaf's open sums, the first tail tokens, the first commits.  Each value
    // is held in a 32-bit register of its own and every load is unconditional behind a
    // uniform test (a missing item re-reads item 0), so no load waits for another; the
    // empty asm makes every load issue before the first store.
    float osk0 = 0.f, osv0 = 0.f, osk1 = 0.f, osv1 = 0.f;
    if (L > 0 && !def0) {
      osk0 = sc.open_k[0][(seq_rows + leaf) * HD + e];
      osv0 = sc.open_v[0][(seq_rows + leaf) * HD + e];
    }
    if (L > 1 && !def1) {
      osk1 = sc.open_k[1][(seq_rows + leaf) * HD + e];
      osv1 = sc.open_v[1][(seq_rows + leaf) * HD + e];
    }
    uint32_t tk[kTailBatch], tvv[kTailBatch];
    if (ntail > 0) {
#pragma unroll
      for (int t = 0; t < kTailBatch; ++t) {
        const size_t src = (seq_rows + sh.pth[t0 + (t < ntail ? t : 0) - P]) * HD + e;
        tk[t] = Bits<T>::ld(k_tree, src);
        tvv[t] = Bits<T>::ld(v_tree, src);
      }
    }
    uint32_t ck[kCommitBatch], cv[kCommitBatch];
    for (int c0 = 0; c0 < ncp; c0 += kCommitBatch) {
#pragma unroll
      for (int t = 0; t < kCommitBatch; ++t) {
        const int i = sh.cp[c0 + t < ncp ? c0 + t : c0];
        const bool l1 = sh.it_l[i] != 0;
        const size_t src = (seq_rows + sh.it_u[i]) * HD + e;
        ck[t] = Bits<T>::ld(l1 ? ek1 : ek0, src);
        cv[t] = Bits<T>::ld(l1 ? ev1 : ev0, src);
      }
      asm volatile("" ::"v"(ck[0]), "v"(ck[1]), "v"(ck[2]), "v"(ck[3]), "v"(ck[4]), "v"(ck[5]), "v"(ck[6]),
                   "v"(ck[7]), "v"(cv[0]), "v"(cv[1]), "v"(cv[2]), "v"(cv[3]), "v"(cv[4]), "v"(cv[5]), "v"(cv[6]),
                   "v"(cv[7]));
#pragma unroll
      for (int t = 0; t < kCommitBatch; ++t)
        if (c0 + t < ncp) {  // uniform
          const int i = sh.cp[c0 + t], j = sh.it_j[i];
          const tv_level& lv = sh.it_l[i] != 0 ? st.lvl[1] : st.lvl[0];
          const size_t tb = sh.it_tile0[i] + (size_t)g * sh.it_gstep[i];
          Bits<T>::st((T*)lv.k, tb + (size_t)(j & 63) * d + dd, ck[t]);
          Bits<T>::st((T*)lv.vt, tb + (size_t)dd * 64 + (j & 63), cv[t]);
        }
    }
    if (def0 || def1) {  // uniform: the deferred levels, from the path tokens
      // the committed open sum counts only while the open block began before the path
      float dk[2], dv[2];
#pragma unroll
      for (int l = 0; l < 2; ++l) {
        const bool on = l == 0 ? def0 : def1;
        const bool open = on && P % st.lvl[l].C != 0;
        dk[l] = open ? st.lvl[l].open_k[(size_t)b * HD + e] : 0.f;
        dv[l] = open ? st.lvl[l].open_v[(size_t)b * HD + e] : 0.f;
      }
      for (int t0 = 0; t0 <= m; t0 += kCommitBatch) {
        uint32_t xk[kCommitBatch], xv[kCommitBatch];
#pragma unroll
        for (int t = 0; t < kCommitBatch; ++t) {  // a batch of path tokens, every load first
          const size_t src = (seq_rows + sh.pth[t0 + t <= m ? t0 + t : t0]) * HD + e;
          xk[t] = Bits<T>::ld(k_tree, src);
          xv[t] = Bits<T>::ld(v_tree, src);
        }
        asm volatile("" ::"v"(xk[0]), "v"(xk[1]), "v"(xk[2]), "v"(xk[3]), "v"(xk[4]), "v"(xk[5]), "v"(xk[6]),
                     "v"(xk[7]), "v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]), "v"(xv[4]), "v"(xv[5]), "v"(xv[6]),
                     "v"(xv[7]));
#pragma unroll
        for (int t = 0; t < kCommitBatch; ++t) {
          if (t0 + t > m) break;  // uniform
          const float fk = Wide<T>::f(xk[t]), fv = Wide<T>::f(xv[t]);
          const int pos = P + t0 + t;
#pragma unroll
          for (int l = 0; l < 2; ++l) {
            if (!(l == 0 ? def0 : def1)) continue;
            dk[l] += fk;
            dv[l] += fv;
            const int C = st.lvl[l].C;
            if ((pos + 1) % C == 0) {  // uniform: the block closes here, its entry is committed
              const int j = pos / C;
              const int i = (l ? nc[0] : 0) + (j - j0[l]);  // its listed block
              const tv_level& lv = l ? st.lvl[1] : st.lvl[0];
              const size_t tb = sh.it_tile0[i] + (size_t)g * sh.it_gstep[i];
              const float cf = (float)C;
              Bits<T>::st((T*)lv.k, tb + (size_t)(j & 63) * d + dd, Wide<T>::bits(dk[l] / cf));
              Bits<T>::st((T*)lv.vt, tb + (size_t)dd * 64 + (j & 63), Wide<T>::bits(dv[l] / cf));
              dk[l] = 0.f;
              dv[l] = 0.f;
            }
          }
        }
      }
      if (def0) {
        osk0 = dk[0];
        osv0 = dv[0];
      }
      if (def1) {
        osk1 = dk[1];
        osv1 = dv[1];
      }
    }
    if (L > 0) {
      st.lvl[0].open_k[(size_t)b * HD + e] = osk0;
      st.lvl[0].open_v[(size_t)b * HD + e] = osv0;
    }
    if (L > 1) {
      st.lvl[1].open_k[(size_t)b * HD + e] = osk1;
      st.lvl[1].open_v[(size_t)b * HD + e] = osv1;
    }
    const size_t tail_row = ((size_t)b * Hkv + g) * (C0 - 1);
    for (int tb0 = 0; tb0 < ntail; tb0 += kTailBatch) {
      if (tb0 > 0) {  // tail tokens past the first batch (C0 > kTailBatch + 1)
#pragma unroll
        for (int t = 0; t < kTailBatch; ++t) {
          const size_t src = (seq_rows + sh.pth[t0 + (tb0 + t < ntail ? tb0 + t : tb0) - P]) * HD + e;
          tk[t] = Bits<T>::ld(k_tree, src);
          tvv[t] = Bits<T>::ld(v_tree, src);
        }
      }
#pragma unroll
      for (int t = 0; t < kTailBatch; ++t)
        if (tb0 + t < ntail) {  // uniform
          const size_t dst = (tail_row + (t0 + tb0 + t - t_new)) * d + dd;
          Bits<T>::st(tail_k, dst, tk[t]);
          Bits<T>::st(tail_v, dst, tvv[t]);
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
  __shared__ RefreshLds sh;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int L = st.n_levels;
  // every read of the inputs and the old counters in one round trip
  const int err = seq_err[b];
  const int m = m_in[b];
  const int P = st.P[b];
  const int pv = tid < D ? path[(size_t)b * D + tid] : -1;
  const uint64_t in_place = sc.in_place != nullptr ? sc.in_place[b] : 0ull;
  if (commit_log != nullptr)
    for (int e = tid; e < L * D * 2; e += nt) commit_log[(size_t)b * L * D * 2 + e] = -1;
  if (tid < D) sh.pth[tid] = pv;
  if (tid == 0) {
    sh.bad = 0;
    sh.ncp = 0;
  }
  __syncthreads();  // log prefill and the reads above happen before any later write
  if (err != TV_SEQ_OK || m < 0) return;
  refresh_body<T>(b, D, st, sc, k_tree, v_tree, m, P, in_place, sh, commit_log, seq_err);
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
  __shared__ RefreshLds sh;
  __shared__ int m_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int L = st.n_levels;
  if (commit_log != nullptr)
    for (int e = tid; e < L * D * 2; e += nt) commit_log[(size_t)b * L * D * 2 + e] = -1;
  const int err = seq_err[b];
  const int P = st.P[b];
  const uint64_t in_place = sc.in_place != nullptr ? sc.in_place[b] : 0ull;
  if (tid < 64) {  // the first wave: every path slot -1, then the accepted path
    if (tid < D) sh.pth[tid] = -1;
    const int m = accept_one(b, D, parents, anc, depth, draft, target, seq_err, m_out, path, bonus, sh.pth);
    if (tid == 0) {
      m_s = m;
      sh.bad = 0;
      sh.ncp = 0;
    }
  }
  __syncthreads();  // the path is in LDS; the log prefill and the reads above are done
  const int m = m_s;
  if (err != TV_SEQ_OK || m < 0) return;
  // slots 0..m hold one node each for a plan from tv_build_tree_mask; refresh_body
  // checks them as it checks a path it is given
  refresh_body<T>(b, D, st, sc, k_tree, v_tree, m, P, in_place, sh, commit_log, seq_err);
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
