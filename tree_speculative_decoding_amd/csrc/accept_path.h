// Greedy accepted-path selection of one draft tree by one wave64, shared by the accept
// kernel and the fused accept + refresh kernel.  TSD-V4 §3.1 (verification yields a
// specific path through the tree, not a prefix length) and §4.4 (accepted-path
// selection after target verify).
//
// Lane i = node i.  A ballot collects the nodes whose draft token equals the target's
// token after their parent; a node is accepted iff its whole chain (its ancestor mask)
// lies inside that ballot.  A wave max over (depth, -index) picks the path end; every
// lane on that chain writes its own slot of the path (slots are the distinct depths
// 0..m).
#pragma once
#include "tv_common.h"

namespace tv {

// Sequence b's acceptance.  seq_err (may be NULL) holds the sequences' status: a flagged
// sequence gets m = -1, bonus = -1 and an all -1 path.  Writes path[b][0..D), m_out[b] and bonus[b]; when pth
// is not NULL (LDS, D entries) the path is also written there.  Returns m to every lane.
__device__ __forceinline__ int accept_one(int b, int D, const int32_t* __restrict__ parents,
                                          const uint64_t* __restrict__ anc, const int32_t* __restrict__ depth,
                                          const int32_t* __restrict__ draft, const int32_t* __restrict__ target,
                                          const int32_t* __restrict__ seq_err, int32_t* __restrict__ m_out,
                                          int32_t* __restrict__ path,
                                          int32_t* __restrict__ bonus, int* pth) {
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)b * D;
  const bool live = lane < D;
  // every load at once, ahead of the status test: the node's chain, depth, parent, draft
  // token and target token (its parent's target and the bonus then come from their lanes)
  uint64_t a = 0;
  int dep = 0, par = -1, dr = 0, tg = -1;
  if (live) {
    a = anc[base + lane] & node_mask(D);
    dep = depth[base + lane];
    par = parents[base + lane];
    dr = draft[base + lane];
    tg = target[base + lane];
  }
  const int err = seq_err != nullptr ? seq_err[b] : TV_SEQ_OK;
  if (err != TV_SEQ_OK) {  // wave-uniform
    if (live) {
      path[base + lane] = -1;
      if (pth != nullptr) pth[lane] = -1;
    }
    if (lane == 0) {
      m_out[b] = -1;
      bonus[b] = -1;
    }
    return -1;
  }
  const bool par_ok = par >= 0 && par < D;
  const int tpar = __shfl(tg, par_ok ? par : 0, 64);
  const bool match = live && (lane == 0 || (par_ok && dr == tpar));
  const uint64_t matched = __ballot(match);
  const bool accepted = live && (a & ~matched) == 0ull;
  // key: deeper wins, then smaller index; root (depth 0, index 0) always qualifies
  const int key = accepted ? ((dep << 8) | (255 - lane)) : -1;
  const int best = wave_max_int(key);
  const int leaf = 255 - (best & 255);
  const int m = best >> 8;
  const uint64_t chain = shfl_u64(a, leaf);
  if (live) {
    if (((chain >> lane) & 1ull) && dep >= 0 && dep < D) {  // (a plan from tv_build_tree_mask: always)
      path[base + dep] = lane;
      if (pth != nullptr) pth[dep] = lane;
    }
    if (lane > m) {
      path[base + lane] = -1;
      if (pth != nullptr) pth[lane] = -1;
    }
  }
  const int bon = __shfl(tg, leaf, 64);
  if (lane == 0) {
    m_out[b] = m;
    bonus[b] = bon;
  }
  return m;
}

}  // namespace tv
