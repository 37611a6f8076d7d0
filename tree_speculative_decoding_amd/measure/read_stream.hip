// Read-stream ceiling of the device's HBM: a plain read-reduce over a large buffer,
// against which the verify attention's achieved bandwidth is also reported (the
// attention kernel is bound by streaming the compressed K/V pools, so the best a plain
// read reaches on the same device is the practical ceiling; MI355X's 8 TB/s is the
// published peak).  A measurement aid only: no step of the verify path runs here.
//
// Grid-stride loop, 16-byte loads, 8 loads in flight per thread before any use; each
// workgroup XORs what it read into one word (so no load can be dropped) and writes it.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(kThreads) void k_read_stream(const uint4* __restrict__ p, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t acc = 0;
  const size_t span = (size_t)kThreads * kInFlight;
  const size_t stride = (size_t)gridDim.x * span;
  size_t i = (size_t)blockIdx.x * span + threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < n16; i += stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int x = 0; x < kInFlight; ++x) v[x] = p[i + (size_t)x * kThreads];
#pragma unroll
    for (int x = 0; x < kInFlight; ++x) acc ^= v[x].x ^ v[x].y ^ v[x].z ^ v[x].w;
  }
  // the ragged end of the buffer (fewer than kInFlight * kThreads chunks in this stride)
  for (; i < n16; i += kThreads) {
    const uint4 v = p[i];
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
// threads on `stream`; workgroup w writes the XOR of the words it read to sink[w] (a
// device buffer of at least `blocks` words).  Returns 0 on success, else the HIP error
// code (-1 for a bad argument; nothing is launched then).
extern "C" __attribute__((visibility("default"))) int tvm_read_stream(const void* p, size_t bytes, int blocks,
                                                                      uint32_t* sink, hipStream_t stream) {
  if (p == nullptr || sink == nullptr || blocks < 1 || bytes % 16 != 0 || ((uintptr_t)p & 15) != 0) return -1;
  hipLaunchKernelGGL(k_read_stream, dim3(blocks), dim3(kThreads), 0, stream, (const uint4*)p, bytes / 16, sink);
  return (int)hipGetLastError();
}
