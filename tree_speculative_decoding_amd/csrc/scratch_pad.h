// Chain-wise compression of every tree node's own branch into the scratch pad (the
// per-node work, shared by the scratch kernel and the prefix kernel's folded workgroups).
// TSD-V4 §4.1 (chains share the prefix state but are compressed independently after
// branching; one compression never mixes two chains) and §4.2 (per-chain compressed
// tokens and intermediate sums stay in the scratch pad until the path is accepted).
//
// Node i sits at position pos = P + depth(i); its block of a level with size C starts at
// b0 = floor(pos/C)*C.  The block sum is the committed open sum (only if b0 < P, i.e. the
// block began before the tree) plus the chain's tokens at positions >= b0, added in chain
// order (root first) in fp32.  A node whose position ends a block writes the entry sum/C
// (rounded once to the element type) and a zero open sum; any other node writes the
// running sum.
//
// In-place chain (TSD-V4 §4.3: with one candidate chain, or when the accepted chain is the
// one already cached, the refresh can be skipped).  When the caller gives
// scratch.in_place, the nodes of one chain -- the path that full acceptance selects, ending
// at the deepest node (smallest index among equals), i.e. the whole tree when it is a
// single chain -- also write the entries they close straight into their pool slots
// (slot j = pos / C >= the committed count, so nothing committed changes and the stream
// never reads them), provided the slot is below the capacity and its page exists; node 0's
// workgroup records that chain in in_place[b].  The refresh then copies only the entries
// of accepted nodes off that chain.  The values are the scratch entries' bits.
//
// The pad depends on the tree tokens, the plan and the committed open sums only, not on
// the prefix: one workgroup per (sequence, node), either in a short kernel of its own
// ahead of the prefix stream or as extra workgroups of the prefix kernel's launch when
// the device has room for them beside the stream.  The tree's depths are in LDS; thread t
// takes the four consecutive elements 4t .. 4t+3 of the node's Hkv*d row (per pass of
// 1024) and walks the node's chain once for every level, issuing the K and V loads of up
// to eight chain nodes before adding them in chain order.  Levels marked in
// scratch.deferred are skipped (no scratch states, no in-place writes).
#pragma once
#include "tv_common.h"

namespace tv {

// Four consecutive elements: loads and stores of 8 (bf16) or 16 (fp32) bytes.
template <typename T> struct Quad;
template <> struct Quad<float> {
  static __device__ __forceinline__ float4 load(const float* p, size_t i) { return *(const float4*)(p + i); }
  static __device__ __forceinline__ void store(float* p, size_t i, float4 v) { *(float4*)(p + i) = v; }
};
template <> struct Quad<uint16_t> {
  static __device__ __forceinline__ float4 load(const uint16_t* p, size_t i) {
    const uint2 r = *(const uint2*)(p + i);
    return make_float4(bf16_bits_to_f32(r.x & 0xffffu), bf16_bits_to_f32(r.x >> 16),
                       bf16_bits_to_f32(r.y & 0xffffu), bf16_bits_to_f32(r.y >> 16));
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float4 v) {
    *(uint2*)(p + i) = make_uint2((uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16),
                                  (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16));
  }
};

// Four consecutive elements as raw bits (8 or 16 bytes), widened to fp32 after the wait.
template <typename T> struct QuadRaw;
template <> struct QuadRaw<float> {
  using type = float4;
  static __device__ __forceinline__ float4 load(const float* p, size_t i) { return *(const float4*)(p + i); }
  static __device__ __forceinline__ float4 widen(float4 r) { return r; }
  static __device__ __forceinline__ void pin(float4 r) { asm volatile("" ::"v"(r.x), "v"(r.y), "v"(r.z), "v"(r.w)); }
};
template <> struct QuadRaw<uint16_t> {
  using type = uint2;
  static __device__ __forceinline__ uint2 load(const uint16_t* p, size_t i) { return *(const uint2*)(p + i); }
  static __device__ __forceinline__ float4 widen(uint2 r) {
    return make_float4(bf16_bits_to_f32(r.x & 0xffffu), bf16_bits_to_f32(r.x >> 16),
                       bf16_bits_to_f32(r.y & 0xffffu), bf16_bits_to_f32(r.y >> 16));
  }
  static __device__ __forceinline__ void pin(uint2 r) { asm volatile("" ::"v"(r.x), "v"(r.y)); }
};

// c ? a : b per component (a select of whole float4 structs is compiled through memory)
__device__ __forceinline__ float4 sel4(bool c, float4 a, float4 b) {
  return make_float4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// LDS of a scratch-pad workgroup: the tree's depths and chains.
struct ScratchLds {
  int dep[TV_MAX_D];
  uint64_t anc[TV_MAX_D];
};

// The scratch pad of node i of sequence b, by one workgroup of 256 threads.  kBatch chain
// nodes' loads are issued together.
template <typename T, int kBatch = 8>
__device__ __forceinline__ void scratch_node(const AttnArgs& a, int b, int i, ScratchLds* sl) {
  const int tid = threadIdx.x;
  // every load that needs no other load's result goes out in one round trip (issued by
  // every lane, without branches): the depths and chains, the status, P, the node's chain
  const int dval = a.depth[(size_t)b * a.anc_ld + (tid < a.D ? tid : 0)];
  const uint64_t aval = a.anc[(size_t)b * a.anc_ld + (tid < a.D ? tid : 0)];
  const int eval = *(a.seq_err != nullptr ? a.seq_err + b : a.P + b);
  const int P = a.P[b];
  const uint64_t chain = a.anc[(size_t)b * a.anc_ld + i] & node_mask(a.D);
  // (an empty use of all of them: the compiler issues them together and waits once,
  // instead of moving each load down to its first use)
  asm volatile("" ::"v"(dval), "v"(eval), "v"(P), "v"((uint32_t)chain), "v"((uint32_t)(chain >> 32)),
               "v"((uint32_t)aval), "v"((uint32_t)(aval >> 32)));
  if (tid < a.D) {
    sl->dep[tid] = dval;
    sl->anc[tid] = aval & node_mask(a.D);
  }
  __syncthreads();
  const bool ok = a.seq_err == nullptr || eval == TV_SEQ_OK;
  uint64_t* in_place = a.scratch.in_place;
  if (!ok) {  // uniform
    if (in_place != nullptr && i == 0 && tid == 0) in_place[b] = 0ull;
    return;
  }
  int* dep_s = sl->dep;
  // the in-place chain: the deepest node, smallest index among equals (every thread scans
  // the depths in LDS), and its chain
  bool on_chain = false;
  if (in_place != nullptr) {
    int leaf = 0;
    for (int u = 1; u < a.D; ++u)
      if (dep_s[u] > dep_s[leaf]) leaf = u;
    const uint64_t lchain = sl->anc[leaf];
    on_chain = (lchain >> i) & 1ull;
    if (i == 0 && tid == 0) in_place[b] = lchain;
  }

  const int pos = P + dep_s[i];
  int b0[TV_MAX_LEVELS];
#pragma unroll
  for (int l = 0; l < TV_MAX_LEVELS; ++l) b0[l] = l < a.n_levels ? (pos / a.C[l]) * a.C[l] : 0;
  const int HD = a.Hkv * a.d;  // a multiple of 64
  const T* kt = (const T*)a.k_tree;
  const T* vt = (const T*)a.v_tree;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);

  using R = QuadRaw<T>;
  static_assert(TV_MAX_LEVELS == 2, "two levels: the sums below are named per level");
  // (a deferred level gets no scratch states: the refresh brings it up to date instead)
  const bool lv1 = a.n_levels > 1 && !((a.scratch.deferred >> 1) & 1u);
  for (int e = 4 * tid; e < HD; e += 4 * 256) {
    // the open sums (level 0's address where level 1 is absent) and the chain's first
    // batch, loaded unconditionally and held as raw bits until every load is out (a
    // selected load is otherwise moved into a branch that waits for it there)
    const size_t so = (size_t)b * HD + e;
    float4 sk0 = *(const float4*)(a.open_k[0] + so), sv0 = *(const float4*)(a.open_v[0] + so);
    float4 sk1 = *(const float4*)(a.open_k[lv1 ? 1 : 0] + so), sv1 = *(const float4*)(a.open_v[lv1 ? 1 : 0] + so);
    // the chain, root first, kBatch nodes at a time: every load of a batch, then the
    // additions in chain order
    uint64_t mm = chain;
    bool first = true;
    do {
      int js[kBatch];
      typename R::type kr[kBatch], vr[kBatch];
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        js[t] = mm != 0ull ? __builtin_ctzll(mm) : -1;
        if (mm != 0ull) mm &= mm - 1ull;
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        const size_t o = ((size_t)b * a.D + (js[t] >= 0 ? js[t] : 0)) * HD + e;
        kr[t] = R::load(kt, o);
        vr[t] = R::load(vt, o);
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        R::pin(kr[t]);
        R::pin(vr[t]);
      }
      if (first) {  // the committed open sums count only where the block began before the tree
        const bool open0 = b0[0] < P, open1 = lv1 && b0[1] < P;
        sk0 = sel4(open0, sk0, z);
        sv0 = sel4(open0, sv0, z);
        sk1 = sel4(open1, sk1, z);
        sv1 = sel4(open1, sv1, z);
        first = false;
      }
#pragma unroll
      for (int t = 0; t < kBatch; ++t) {
        if (js[t] < 0) continue;  // (the rest of the batch is empty too)
        const int pj = P + dep_s[js[t]];
        const float4 kk = R::widen(kr[t]), vv = R::widen(vr[t]);
        if (pj >= b0[0]) {
          sk0 = add4(sk0, kk);
          sv0 = add4(sv0, vv);
        }
        if (lv1 && pj >= b0[1]) {
          sk1 = add4(sk1, kk);
          sv1 = add4(sv1, vv);
        }
      }
    } while (mm != 0ull);
#pragma unroll
    for (int l = 0; l < TV_MAX_LEVELS; ++l) {
      if (l >= a.n_levels || ((a.scratch.deferred >> l) & 1u)) continue;
      const float4 ks = sel4(l != 0, sk1, sk0), vs = sel4(l != 0, sv1, sv0);  // (l is a constant here)
      const int C = a.C[l];
      const size_t dst = ((size_t)b * a.D + i) * HD + e;
      if ((pos + 1) % C == 0) {
        const float cf = (float)C;
        const float4 ek = make_float4(ks.x / cf, ks.y / cf, ks.z / cf, ks.w / cf);
        const float4 ev = make_float4(vs.x / cf, vs.y / cf, vs.z / cf, vs.w / cf);
        Quad<T>::store((T*)a.scratch.entry_k[l], dst, ek);
        Quad<T>::store((T*)a.scratch.entry_v[l], dst, ev);
        *(float4*)(a.scratch.open_k[l] + dst) = z;
        *(float4*)(a.scratch.open_v[l] + dst) = z;
        const int j = pos / C;  // the pool slot this block would be committed to
        if (on_chain && j < a.cap[l]) {  // uniform
          const bool paged = a.pt[l] != nullptr;
          int page = 0;
          if (paged) page = a.pt[l][(size_t)b * a.ppseq[l] + (j >> 6)];
          if (!paged || (page >= 0 && page < a.npages[l])) {
            const int g = e / a.d, c = e - g * a.d;  // four channels of one head
            const size_t tb = tile_offset(paged, page, a.cap[l], a.B, a.Hkv, a.d, b, g, j >> 6);
            Quad<T>::store((T*)a.pk[l], tb + (size_t)(j & 63) * a.d + c, ek);
            T* vt = (T*)a.pvt[l] + tb + (size_t)c * 64 + (j & 63);
            Elem<T>::store(vt, 0, ev.x);
            Elem<T>::store(vt, 64, ev.y);
            Elem<T>::store(vt, 128, ev.z);
            Elem<T>::store(vt, 192, ev.w);
          }
        }
      } else {
        *(float4*)(a.scratch.open_k[l] + dst) = ks;
        *(float4*)(a.scratch.open_v[l] + dst) = vs;
      }
    }
  }
}

}  // namespace tv
