// Verify preprocess: parent array -> per-node chain bitmask and depth.
// TSD-V4 §4.1 (the verification plan describes the candidate chains and their
// compression boundaries) and §4.3 (plan metadata is prepared on the device).
//
// One wave64 per sequence, lane i = node i.  Validity is one ballot; the chain of
// every node is built by pointer jumping over the parent links held in registers:
// after round r each lane's mask covers its ancestors within distance 2^r - 1, so
// six rounds cover any tree of <= 64 nodes.  depth = popcount(mask) - 1.
#include "tv_launch.h"

namespace tv {

__global__ __launch_bounds__(256) void k_tree_mask(int B, int D, const int32_t* __restrict__ parents,
                                                   uint64_t* __restrict__ anc, int32_t* __restrict__ depth,
                                                   int32_t* __restrict__ seq_err) {
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (b >= B) return;  // whole wave leaves together
  const bool live = lane < D;
  const int p = live ? parents[(size_t)b * D + lane] : 0;
  const bool bad = live && (lane == 0 ? p != -1 : (p < 0 || p >= lane));
  const bool any_bad = __ballot(bad) != 0ull;

  uint64_t mask = live ? (1ull << lane) : 0ull;
  int jump = (live && lane > 0 && !any_bad) ? p : -1;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = jump < 0 ? lane : jump;
    const uint64_t m_src = shfl_u64(mask, src);
    const int j_src = __shfl(jump, src, 64);
    if (jump >= 0) {
      mask |= m_src;
      jump = j_src;
    }
  }
  if (live) {
    const size_t o = (size_t)b * D + lane;
    anc[o] = any_bad ? 0ull : mask;
    depth[o] = any_bad ? 0 : (__popcll(mask) - 1);
  }
  if (lane == 0) seq_err[b] = any_bad ? TV_SEQ_BAD_PARENT : TV_SEQ_OK;
}

hipError_t launch_tree_mask(int B, int D, const int32_t* parents, uint64_t* anc, int32_t* depth,
                            int32_t* seq_err, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int waves_per_block = 4;
  dim3 grid((B + waves_per_block - 1) / waves_per_block);
  hipLaunchKernelGGL(k_tree_mask, grid, dim3(64 * waves_per_block), 0, s, B, D, parents, anc, depth,
                     seq_err);
  return hipGetLastError();
}

}  // namespace tv
