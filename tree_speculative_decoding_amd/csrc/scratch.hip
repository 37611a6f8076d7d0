// The scratch pad kernel: one workgroup per (sequence, node) (scratch_node, in
// scratch_pad.h), launched ahead of the prefix stream unless the prefix kernel builds the
// pad in workgroups of its own launch.  TSD-V4 §4.1, §4.2.
#include "scratch_pad.h"
#include "tv_launch.h"

namespace tv {

template <typename T>
__global__ __launch_bounds__(256) void k_scratch(AttnArgs a) {
  __shared__ ScratchLds sl;
  const int b = blockIdx.x / a.D;
  scratch_node<T>(a, b, blockIdx.x - b * a.D, &sl);
}

hipError_t launch_scratch(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.n_levels == 0 || !a.build_scratch) return hipSuccess;
  dim3 grid(a.B * a.D), block(256);
  if (a.dtype == TV_BF16)
    hipLaunchKernelGGL(k_scratch<uint16_t>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_scratch<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace tv
