// Greedy accepted-path selection: one wave64 per sequence (accept_one, in
// accept_path.h).  TSD-V4 §3.1, §4.4.
#include "accept_path.h"
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
  const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (b >= B) return;
  accept_one(b, D, parents, anc, depth, draft, target, seq_err, m_out, path, bonus, nullptr);
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
