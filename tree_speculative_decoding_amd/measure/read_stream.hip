// Read-stream ceiling of the device's HBM: a plain read-reduce over a large buffer,
// against which the verify attention's achieved bandwidth is also reported (the
// attention kernel is bound by streaming the compressed K/V pools, so the best a plain
// read reaches on the same device is the practical ceiling; MI355X's 8 TB/s is the
// published peak).  A measurement aid only: no step of the verify path runs here.
//
// Grid-stride loop, 16-byte loads, 8 loads in flight per thread before any use; each
// workgroup XORs what it read into one word (so no load can be dropped) and writes it.
// The loads are plain or carry the nontemporal hint (the verify kernel streams its pools
// with the hint; on MI355X the hinted read is the faster one).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if (kNT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool kNT>
__global__ __launch_bounds__(kThreads) void k_read_stream(const u32x4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t acc = 0;
  const size_t span = (size_t)kThreads * kInFlight;
  const size_t stride = (size_t)gridDim.x * span;
  size_t i = (size_t)blockIdx.x * span + threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < n16; i += stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int x = 0; x < kInFlight; ++x) v[x] = load16<kNT>(p + i + (size_t)x * kThreads);
#pragma unroll
    for (int x = 0; x < kInFlight; ++x) acc ^= v[x].x ^ v[x].y ^ v[x].z ^ v[x].w;
  }
  // the ragged end of the buffer (fewer than kInFlight * kThreads chunks in this stride)
  for (; i < n16; i += kThreads) {
    const u32x4 v = load16<kNT>(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r ^= red[w];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device buffer `p` with `blocks` workgroups of 256
// threads on `stream`, with nontemporal loads when `nontemporal` is nonzero; workgroup w
// writes the XOR of the words it read to sink[w] (a device buffer of at least `blocks`
// words).  Returns 0 on success, else the HIP error code (-1 for a bad argument; nothing
// is launched then).
extern "C" __attribute__((visibility("default"))) int tvm_read_stream(const void* p, size_t bytes, int blocks,
                                                                      int nontemporal, uint32_t* sink,
                                                                      hipStream_t stream) {
  if (p == nullptr || sink == nullptr || blocks < 1 || bytes % 16 != 0 || ((uintptr_t)p & 15) != 0) return -1;
  if (nontemporal)
    hipLaunchKernelGGL(k_read_stream<true>, dim3(blocks), dim3(kThreads), 0, stream, (const u32x4*)p, bytes / 16, sink);
  else
    hipLaunchKernelGGL(k_read_stream<false>, dim3(blocks), dim3(kThreads), 0, stream, (const u32x4*)p, bytes / 16, sink);
  return (int)hipGetLastError();
}
