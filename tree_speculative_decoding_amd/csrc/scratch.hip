// Chain-wise compression of every tree node's own branch into the scratch pad.
// TSD-V4 §4.1 (chains share the prefix state but are compressed independently
// after branching; one compression never mixes two chains) and §4.2 (per-chain
// compressed tokens and intermediate sums stay in the scratch pad until the path
// is accepted).
//
// One workgroup per (sequence, node); threads over (KV head, channel).  Node i
// sits at position pos = P + depth(i); its block of a level with size C starts at
// b0 = floor(pos/C)*C.  The block sum is the committed open sum (only if b0 < P,
// i.e. the block began before the tree) plus the chain's tokens at positions
// >= b0, added in chain order in fp32.  A node whose position ends a block
// writes the entry sum/C (rounded once to the element type) and a zero open
// sum; any other node writes the running sum.
#include "tv_common.h"

namespace tv {

template <typename T>
__global__ __launch_bounds__(256) void k_scratch(AttnArgs a) {
  const int b = blockIdx.x / a.D;
  const int i = blockIdx.x - b * a.D;
  if (a.seq_err != nullptr && a.seq_err[b] != TV_SEQ_OK) return;
  const int P = a.P[b];
  const uint64_t chain = a.anc[(size_t)b * a.D + i] & node_mask(a.D);
  const int pos = P + a.depth[(size_t)b * a.D + i];
  const int HD = a.Hkv * a.d;
  const T* kt = (const T*)a.k_tree;
  const T* vt = (const T*)a.v_tree;
  for (int l = 0; l < a.n_levels; ++l) {
    const int C = a.C[l];
    const int b0 = (pos / C) * C;
    const bool closes = (pos + 1) % C == 0;
    for (int e = threadIdx.x; e < HD; e += blockDim.x) {
      const size_t so = (size_t)b * HD + e;
      float sk = b0 < P ? a.open_k[l][so] : 0.f;
      float sv = b0 < P ? a.open_v[l][so] : 0.f;
      uint64_t mm = chain;
      while (mm != 0ull) {
        const int u = __builtin_ctzll(mm);
        mm &= mm - 1ull;
        if (P + a.depth[(size_t)b * a.D + u] >= b0) {
          const size_t o = ((size_t)b * a.D + u) * HD + e;
          sk += Elem<T>::load(kt, o);
          sv += Elem<T>::load(vt, o);
        }
      }
      const size_t dst = ((size_t)b * a.D + i) * HD + e;
      if (closes) {
        Elem<T>::store((T*)a.scratch.entry_k[l], dst, sk / (float)C);
        Elem<T>::store((T*)a.scratch.entry_v[l], dst, sv / (float)C);
        a.scratch.open_k[l][dst] = 0.f;
        a.scratch.open_v[l][dst] = 0.f;
      } else {
        a.scratch.open_k[l][dst] = sk;
        a.scratch.open_v[l][dst] = sv;
      }
    }
  }
}

hipError_t launch_scratch(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.n_levels == 0) return hipSuccess;
  dim3 grid(a.B * a.D), block(256);
  if (a.dtype == TV_BF16)
    hipLaunchKernelGGL(k_scratch<uint16_t>, grid, block, 0, s, a);
  else
    hipLaunchKernelGGL(k_scratch<float>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace tv
