// Branch-aware verify attention, final step: merge the split-KV partials of the
// shared prefix, add the finest level's raw tail and the node's own chain, and
// normalise.  TSD-V4 §3.1: a candidate sees the accepted context and the
// ancestors along its own branch, never candidates of other branches.
//
// One wave64 per query row (sequence, node, head); each lane owns d/64 output
// channels.  The chain is the node's ancestor mask: only its set bits are read,
// so K/V of other branches never enter the arithmetic (excluded by selection,
// not by a -inf score).  Everything is combined with the same base-2 online
// softmax as the prefix kernels.
#include "tv_common.h"

namespace tv {

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  constexpr int EPL = DH / 64;
  const int lane = threadIdx.x & 63;
  const long row_id = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const long n_rows = (long)a.B * a.D * a.Hq;
  if (row_id >= n_rows) return;
  const int h = (int)(row_id % a.Hq);
  const int i = (int)((row_id / a.Hq) % a.D);
  const int b = (int)(row_id / ((long)a.Hq * a.D));
  const int g = h / a.G;
  const int r = i * a.G + (h - g * a.G);
  const size_t obase = (((size_t)b * a.D + i) * a.Hq + h) * DH + lane * EPL;
  T* out = (T*)a.out;

  if (a.seq_err != nullptr && a.seq_err[b] != TV_SEQ_OK) {
#pragma unroll
    for (int x = 0; x < EPL; ++x) Elem<T>::store(out, obase + x, 0.f);
    if (a.lse != nullptr && lane == 0) a.lse[((size_t)b * a.D + i) * a.Hq + h] = -INFINITY;
    return;
  }

  float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) o[x] = 0.f;

  // partials of the shared prefix: one per workgroup whose slice touched this row's unit
  const size_t bg = (size_t)b * a.Hkv + g;
  const long long u = (long long)bg * a.row_blocks + r / 64;
  const int n_parts = a.parts > 0 ? unit_part_count(u, a.tmax, a.per) : 0;
  for (int s = 0; s < n_parts; ++s) {
    const size_t wrow = (bg * a.smax + s) * a.R + r;
    const float2 ml = a.ws_ml[wrow];
    if (ml.y > 0.f) {
      const float mn = fmaxf(m, ml.x);
      const float ca = exp2f(m - mn), cb = exp2f(ml.x - mn);
      l = l * ca + ml.y * cb;
#pragma unroll
      for (int x = 0; x < EPL; ++x) o[x] = o[x] * ca + a.ws_o[wrow * DH + lane * EPL + x] * cb;
      m = mn;
    }
  }

  const T* q = (const T*)a.q;
  float qv[EPL];
#pragma unroll
  for (int x = 0; x < EPL; ++x) qv[x] = Elem<T>::load(q, obase + x);

  auto absorb = [&](const T* kr, const T* vr) {
    float part = 0.f;
#pragma unroll
    for (int x = 0; x < EPL; ++x) part = fmaf(qv[x], Elem<T>::load(kr, lane * EPL + x), part);
    const float sc = wave_sum(part) * a.scale_log2;
    const float mn = fmaxf(m, sc);
    const float ca = exp2f(m - mn), cb = exp2f(sc - mn);
    l = l * ca + cb;
#pragma unroll
    for (int x = 0; x < EPL; ++x) o[x] = o[x] * ca + Elem<T>::load(vr, lane * EPL + x) * cb;
    m = mn;
  };

  // raw tokens of the finest level's open block
  if (a.n_levels > 0 && a.C[0] > 1) {
    const int C0 = a.C[0];
    const int rr = a.P[b] % C0;
    const T* tk = (const T*)a.tail_k;
    const T* tv_ = (const T*)a.tail_v;
    for (int t = 0; t < rr; ++t) {
      const size_t off = (bg * (C0 - 1) + t) * DH;
      absorb(tk + off, tv_ + off);
    }
  }
  // the node's own chain: ancestors and itself
  uint64_t chain = a.anc[(size_t)b * a.D + i] & node_mask(a.D);
  const T* kt = (const T*)a.k_tree;
  const T* vt = (const T*)a.v_tree;
  while (chain != 0ull) {
    const int j = __builtin_ctzll(chain);
    chain &= chain - 1ull;
    const size_t off = (((size_t)b * a.D + j) * a.Hkv + g) * DH;
    absorb(kt + off, vt + off);
  }

  const float inv = 1.0f / l;
#pragma unroll
  for (int x = 0; x < EPL; ++x) Elem<T>::store(out, obase + x, o[x] * inv);
  if (a.lse != nullptr && lane == 0)
    a.lse[((size_t)b * a.D + i) * a.Hq + h] = (m + log2f(l)) * kLn2;
}

hipError_t launch_attn_merge(const AttnArgs& a, hipStream_t s) {
  const long rows = (long)a.B * a.D * a.Hq;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (a.dtype == TV_BF16) {
    if (a.d == 128)
      hipLaunchKernelGGL((k_attn_merge<uint16_t, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_merge<uint16_t, 64>), grid, block, 0, s, a);
  } else {
    if (a.d == 128)
      hipLaunchKernelGGL((k_attn_merge<float, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_attn_merge<float, 64>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace tv
