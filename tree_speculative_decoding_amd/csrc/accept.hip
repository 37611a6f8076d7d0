// Greedy accepted-path selection.  TSD-V4 §3.1 (verification yields a specific
// path through the tree, not a prefix length) and §4.4 (accepted-path selection
// after target verify).
//
// One wave64 per sequence, lane i = node i.  A ballot collects the nodes whose
// draft token equals the target's token after their parent; a node is accepted
// iff its whole chain (its ancestor mask) lies inside that ballot.  A wave max
// over (depth, -index) picks the path end; every lane on that chain writes its
// own slot of the path (slots are the distinct depths 0..m).
#include "tv_launch.h"

namespace tv {

__global__ __launch_bounds__(256) void k_accept(int B, int D, const int32_t* __restrict__ parents,
                                                const uint64_t* __restrict__ anc,
                                                const int32_t* __restrict__ depth,
                                                const int32_t* __restrict__ draft,
                                                const int32_t* __restrict__ target,
                                                const int32_t* __restrict__ seq_err,
                                                int32_t* __restrict__ m_out, int32_t* __restrict__ path,
                                                int32_t* __restrict__ bonus) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (b >= B) return;
  const size_t base = (size_t)b * D;
  const bool live = lane < D;
  if (seq_err != nullptr && seq_err[b] != TV_SEQ_OK) {
    if (live) path[base + lane] = -1;
    if (lane == 0) {
      m_out[b] = -1;
      bonus[b] = -1;
    }
    return;
  }
  bool match = false;
  uint64_t a = 0;
  int dep = 0;
  if (live) {
    a = anc[base + lane] & node_mask(D);
    dep = depth[base + lane];
    if (lane == 0) {
      match = true;
    } else {
      const int p = parents[base + lane];
      match = p >= 0 && p < D && draft[base + lane] == target[base + p];
    }
  }
  const uint64_t matched = __ballot(match);
  const bool accepted = live && (a & ~matched) == 0ull;
  // key: deeper wins, then smaller index; root (depth 0, index 0) always qualifies
  const int key = accepted ? ((dep << 8) | (255 - lane)) : -1;
  const int best = wave_max_int(key);
  const int leaf = 255 - (best & 255);
  const int m = best >> 8;
  const uint64_t chain = shfl_u64(a, leaf);
  if (live) {
    if ((chain >> lane) & 1ull) path[base + dep] = lane;
    if (lane > m) path[base + lane] = -1;
  }
  if (lane == 0) {
    m_out[b] = m;
    bonus[b] = target[base + leaf];
  }
}

hipError_t launch_accept(int B, int D, const int32_t* parents, const uint64_t* anc,
                         const int32_t* depth, const int32_t* draft, const int32_t* target,
                         const int32_t* seq_err, int32_t* m, int32_t* path, int32_t* bonus,
                         hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int waves_per_block = 4;
  dim3 grid((B + waves_per_block - 1) / waves_per_block);
  hipLaunchKernelGGL(k_accept, grid, dim3(64 * waves_per_block), 0, s, B, D, parents, anc, depth,
                     draft, target, seq_err, m, path, bonus);
  return hipGetLastError();
}

}  // namespace tv
