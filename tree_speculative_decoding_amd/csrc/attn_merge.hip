// Branch-aware verify attention, final step (TSD-V4 §3.1: a candidate sees the accepted
// context and the ancestors on its own branch, never candidates of other branches):
// merge the prefix-stream partials of a query row (weights 2^(m_s - M) over the row's
// slices, slices with an empty sum weighing nothing, by selection), and normalise.
//
// k_attn_merge: the MFMA path, whose prefix kernel already attended the raw tail and the
// chain; a row's slices spread over groups of 32 threads, every load of a thread in one
// round, the groups combined through LDS (see the kernel).
//
// k_attn_finish: every other path (the fp32 vector kernel, d = 64, trees whose tail +
// tree chunk exceeds 64 entries).  One workgroup of 4 waves per (sequence, KV head, 4
// rows of a unit's block of unit_rows = 64 or 128 query rows), one wave per query row
// r = node * G + head-in-group, each lane d/64 channels of the row.  The partials of a
// row are merged across lanes, not one after another: the lanes read the slices' (max,
// sum) pairs together and reduce the common maximum M, then the partial rows are read 16
// at a time (nontemporal after long slices) with no load waiting on another.  Then the
// finest level's raw tail and the node's own chain: the D tree tokens of the KV head are
// staged in LDS, and the chain is the node's ancestor mask: only its set bits are read,
// so K/V of other branches never enter the arithmetic (excluded by selection, not by a
// -inf score).  Chain scores are reduced eight at a time with interleaved shuffles, then
// folded into the same base-2 online softmax as the prefix kernels.
#include "tv_launch.h"

namespace tv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFinishWaves = 4;   // rows per workgroup
constexpr int kMergeBatch = 16;   // partial rows read together

// NT: the partials are read with the nontemporal hint (they were written with it).
template <typename T, int DH, bool NT>
__global__ __launch_bounds__(kFinishWaves * 64) void k_attn_finish(AttnArgs a) {
  constexpr int EPL = DH / 64;  // channels per lane
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  T* kt_s = (T*)lds_raw;                         // [D][DH]
  T* vt_s = kt_s + (size_t)a.D * DH;             // [D][DH]

  const int groups = a.unit_rows / kFinishWaves;  // workgroups per unit's rows
  const int g = blockIdx.x % a.Hkv;
  const int rb = blockIdx.x / a.Hkv / groups;
  const int rg = blockIdx.x / a.Hkv % groups;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const size_t bg = (size_t)b * a.Hkv + g;
  const bool bad = a.seq_err != nullptr && a.seq_err[b] != TV_SEQ_OK;
  T* out = (T*)a.out;

  if (!a.fused_tree) {  // stage the tree tokens of this KV head
    const T* ktg = (const T*)a.k_tree;
    const T* vtg = (const T*)a.v_tree;
    for (int e = tid; e < a.D * DH; e += blockDim.x) {
      const int j = e / DH, c = e - j * DH;
      const size_t o = (((size_t)b * a.D + j) * a.Hkv + g) * DH + c;
      kt_s[e] = ktg[o];
      vt_s[e] = vtg[o];
    }
    __syncthreads();
  }

  const uint64_t nodes = node_mask(a.D);
  const T* q = (const T*)a.q;
  {
    const int r = rb * a.unit_rows + rg * kFinishWaves + w;
    if (r >= a.R) return;  // wave-uniform; no barrier follows
    const int i = r / a.G, hh = r - i * a.G, h = g * a.G + hh;
    const size_t obase = (((size_t)b * a.D + i) * a.Hq + h) * DH + lane * EPL;
    if (bad) {
#pragma unroll
      for (int x = 0; x < EPL; ++x) Elem<T>::store(out, obase + x, 0.f);
      if (a.lse != nullptr && lane == 0) a.lse[((size_t)b * a.D + i) * a.Hq + h] = -INFINITY;
      return;
    }
    // partials of the shared prefix: one per workgroup whose slice touched this unit
    const int u = (int)bg * a.row_blocks + rb;
    const int n_parts = a.parts > 0 ? unit_part_count(a, u) : 0;
    const int p0 = a.parts > 0 ? unit_first_part(a, u) : 0;
    // with the tail and chain attended by the prefix kernel, a unit it covered with one
    // workgroup is already written; otherwise its partials already hold tail and chain
    if (a.fused_tree && n_parts == 1) return;
    float m = -INFINITY, l = 0.f, o[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) o[x] = 0.f;
    // slice s of this row (workgroup p0 + s, pair p0 + s + u): row0 + s * unit_rows
    const size_t row0 = partial_row(a, p0, u, r - rb * a.unit_rows);
    const size_t sstride = (size_t)a.unit_rows;
    // (max, sum) of slice s0 + lane; lanes past the last slice read the last one's and
    // drop it by selection
    auto slice_ml = [&](int s0) {
      const int s = min(s0 + lane, n_parts - 1);
      const f32x2* src = (const f32x2*)(a.ws_ml + row0 + (size_t)s * sstride);
      const f32x2 mlv = NT ? __builtin_nontemporal_load(src) : *src;
      float2 ml = make_float2(mlv.x, mlv.y);
      asm volatile("" ::"v"(ml.x), "v"(ml.y));
      if (s0 + lane >= n_parts) ml.y = 0.f;
      return ml;
    };
    float2 ml0 = make_float2(-INFINITY, 0.f);
    float M = -INFINITY;
    for (int s0 = 0; s0 < n_parts; s0 += 64) {
      const float2 ml = slice_ml(s0);
      if (s0 == 0) ml0 = ml;
      if (ml.y > 0.f) M = fmaxf(M, ml.x);
    }
    M = wave_max(M);
    if (M != -INFINITY) {  // wave-uniform: some slice saw a visible entry
      float L = 0.f;
      for (int s0 = 0; s0 < n_parts; s0 += 64) {
        const float2 ml = s0 == 0 ? ml0 : slice_ml(s0);
        const float c = ml.y > 0.f ? exp2f(ml.x - M) : 0.f;
        L = fmaf(c, ml.y, L);
        const int cnt = min(64, n_parts - s0);
        for (int t0 = 0; t0 < cnt; t0 += kMergeBatch) {
          float v[kMergeBatch][EPL], ct[kMergeBatch];
#pragma unroll
          for (int t = 0; t < kMergeBatch; ++t) {
            const int tt = min(t0 + t, cnt - 1);  // in range; weight 0 past cnt
            ct[t] = t0 + t < cnt ? __shfl(c, tt, 64) : 0.f;
            const float* src = a.ws_o + (row0 + (size_t)(s0 + tt) * sstride) * DH + lane * EPL;
#pragma unroll
            for (int x = 0; x < EPL; ++x) v[t][x] = NT ? __builtin_nontemporal_load(src + x) : src[x];
          }
          // every load above is issued before any is used (none may move under the
          // selections below)
#pragma unroll
          for (int t = 0; t < kMergeBatch; ++t)
#pragma unroll
            for (int x = 0; x < EPL; ++x) asm volatile("" ::"v"(v[t][x]));
#pragma unroll
          for (int t = 0; t < kMergeBatch; ++t)
#pragma unroll
            for (int x = 0; x < EPL; ++x) o[x] = ct[t] > 0.f ? fmaf(ct[t], v[t][x], o[x]) : o[x];
        }
      }
      m = M;
      l = wave_sum(L);
    }

    float qv[EPL];
#pragma unroll
    for (int x = 0; x < EPL; ++x) qv[x] = Elem<T>::load(q, obase + x);

    // raw tokens of the finest level's open block (at most C0 - 1 of them)
    if (!a.fused_tree && a.n_levels > 0 && a.C[0] > 1) {
      const int C0 = a.C[0];
      const int rr = a.P[b] % C0;
      const T* tk = (const T*)a.tail_k;
      const T* tvv = (const T*)a.tail_v;
      for (int t = 0; t < rr; ++t) {
        const size_t off = (bg * (C0 - 1) + t) * DH + lane * EPL;
        float part = 0.f;
#pragma unroll
        for (int x = 0; x < EPL; ++x) part = fmaf(qv[x], Elem<T>::load(tk, off + x), part);
        const float sc = wave_sum(part) * a.scale_log2;
        const float mn = fmaxf(m, sc);
        const float ca = exp2f(m - mn), cb = exp2f(sc - mn);
        l = l * ca + cb;
#pragma unroll
        for (int x = 0; x < EPL; ++x) o[x] = o[x] * ca + Elem<T>::load(tvv, off + x) * cb;
        m = mn;
      }
    }

    // the node's own chain (ancestors and itself), eight nodes per round
    uint64_t chain = a.fused_tree ? 0ull : a.anc[(size_t)b * a.anc_ld + i] & nodes;
    while (chain != 0ull) {
      int nj[8];
      float sc[8];
      int cnt = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        nj[t] = chain != 0ull ? __builtin_ctzll(chain) : -1;
        if (chain != 0ull) {
          chain &= chain - 1ull;
          ++cnt;
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float part = 0.f;
        if (nj[t] >= 0) {
#pragma unroll
          for (int x = 0; x < EPL; ++x)
            part = fmaf(qv[x], Elem<T>::load(kt_s, (size_t)nj[t] * DH + lane * EPL + x), part);
        }
        sc[t] = part;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int t = 0; t < 8; ++t) sc[t] += __shfl_xor(sc[t], off, 64);
      float mx = m;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        sc[t] *= a.scale_log2;
        if (t < cnt) mx = fmaxf(mx, sc[t]);
      }
      const float ca = exp2f(m - mx);
      l *= ca;
#pragma unroll
      for (int x = 0; x < EPL; ++x) o[x] *= ca;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t < cnt) {
          const float p = exp2f(sc[t] - mx);
          l += p;
#pragma unroll
          for (int x = 0; x < EPL; ++x)
            o[x] = fmaf(p, Elem<T>::load(vt_s, (size_t)nj[t] * DH + lane * EPL + x), o[x]);
        }
      }
      m = mx;
    }

    const float inv = 1.0f / l;
#pragma unroll
    for (int x = 0; x < EPL; ++x) Elem<T>::store(out, obase + x, o[x] * inv);
    if (a.lse != nullptr && lane == 0) a.lse[((size_t)b * a.D + i) * a.Hq + h] = (m + log2f(l)) * kLn2;
  }
}

// The merge of split units on the MFMA path, whose prefix kernel already attended the raw
// tail and the chain and wrote the rows of whole units itself: a unit's row of n slices is
// spread over SG groups of 32 threads (slices sg, sg + SG, ...; each thread 4 channels), so
// every (max, sum) pair and partial row the thread needs (at most JR) is loaded in one round
// before any is used; the groups of a row combine their maxima, then their weighted sums,
// through LDS in group order.  8 / SG rows per 256-thread workgroup.  The summation order
// depends only on n and SG, so results do not depend on timing.  Rows of more than SG * JR
// slices (only with very many workgroups per unit) read the rest in further rounds.
template <int SG, int JR, bool NT>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  constexpr int DH = 128;
  constexpr int RPW = 8 / SG;  // rows per workgroup
  __shared__ float red_m[8], red_l[8];
  __shared__ __attribute__((aligned(16))) f32x4 red_o[8][DH / 4];

  const int tid = threadIdx.x, lane = tid & 31, grp = tid >> 5;
  const int slot = grp / SG, sg = grp - slot * SG;
  const int groups = a.unit_rows / RPW;  // workgroups per unit
  const int g = blockIdx.x % a.Hkv;
  const int rb = blockIdx.x / a.Hkv / groups;
  const int rg = blockIdx.x / a.Hkv % groups;
  const int b = blockIdx.y;
  const int u = (b * a.Hkv + g) * a.row_blocks + rb;
  const int n = unit_part_count(a, u);
  if (n == 1) return;  // a whole unit (uniform): the prefix kernel wrote its rows
  const int lrow = rg * RPW + slot;       // row within the unit
  const int r = rb * a.unit_rows + lrow;  // row r = node * G + head-in-group of KV head g
  const bool valid = r < a.R;             // (the workspace holds every row of a unit: in bounds)
  const int32_t st = a.seq_err != nullptr ? a.seq_err[b] : TV_SEQ_OK;
  const size_t row0 = partial_row(a, unit_first_part(a, u), u, lrow);  // slice s: row0 + s * unit_rows
  const int JT = (n + SG - 1) / SG;  // slices per group, rounded up

  auto ld_o = [&](int s) -> f32x4 {
    const f32x4* p = (const f32x4*)(a.ws_o + (row0 + (size_t)s * a.unit_rows) * DH) + lane;
    return NT ? __builtin_nontemporal_load(p) : *p;
  };
  auto ld_ml = [&](int s) -> f32x2 {
    const f32x2* p = (const f32x2*)(a.ws_ml + row0 + (size_t)s * a.unit_rows);
    return NT ? __builtin_nontemporal_load(p) : *p;
  };
  // first round: slices sg + j * SG (j < JR), past n clamped to the last and weighed 0
  f32x4 ov[JR];
  f32x2 mlv[JR];
#pragma unroll
  for (int j = 0; j < JR; ++j) {
    const int s = min(sg + j * SG, n - 1);
    ov[j] = ld_o(s);
    mlv[j] = ld_ml(s);
  }
  // every load above is issued before any is used
#pragma unroll
  for (int j = 0; j < JR; ++j) asm volatile("" ::"v"(ov[j]), "v"(mlv[j]));
  float mt = -INFINITY;
#pragma unroll
  for (int j = 0; j < JR; ++j)
    if (sg + j * SG < n && mlv[j].y > 0.f) mt = fmaxf(mt, mlv[j].x);
  for (int j = JR; j < JT; ++j) {  // further rounds (rare): their maxima
    const int s = sg + j * SG;
    if (s < n) {
      const f32x2 ml = ld_ml(s);
      if (ml.y > 0.f) mt = fmaxf(mt, ml.x);
    }
  }
  float M = mt;
  if (SG > 1) {
    if (lane == 0) red_m[grp] = mt;
    __syncthreads();
    M = red_m[slot * SG];
#pragma unroll
    for (int i = 1; i < SG; ++i) M = fmaxf(M, red_m[slot * SG + i]);
  }
  // weighted sums in slice order: weights 2^(m_s - M), empty slices weigh nothing
  f32x4 ot = f32x4{0.f, 0.f, 0.f, 0.f};
  float lt = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < JR; ++j) {
      const float c = sg + j * SG < n && mlv[j].y > 0.f ? exp2f(mlv[j].x - M) : 0.f;
      if (c > 0.f) {
        lt = fmaf(c, mlv[j].y, lt);
        ot[0] = fmaf(c, ov[j][0], ot[0]);
        ot[1] = fmaf(c, ov[j][1], ot[1]);
        ot[2] = fmaf(c, ov[j][2], ot[2]);
        ot[3] = fmaf(c, ov[j][3], ot[3]);
      }
    }
    for (int j = JR; j < JT; ++j) {
      const int s = sg + j * SG;
      if (s < n) {
        const f32x2 ml = ld_ml(s);
        if (ml.y > 0.f) {
          const float c = exp2f(ml.x - M);
          const f32x4 o = ld_o(s);
          lt = fmaf(c, ml.y, lt);
          ot[0] = fmaf(c, o[0], ot[0]);
          ot[1] = fmaf(c, o[1], ot[1]);
          ot[2] = fmaf(c, o[2], ot[2]);
          ot[3] = fmaf(c, o[3], ot[3]);
        }
      }
    }
  }
  if (SG > 1) {
    red_o[grp][lane] = ot;
    if (lane == 0) red_l[grp] = lt;
    __syncthreads();
    if (sg != 0) return;
    ot = red_o[slot * SG][lane];
    lt = red_l[slot * SG];
#pragma unroll
    for (int i = 1; i < SG; ++i) {
      const f32x4 o = red_o[slot * SG + i][lane];
      ot[0] += o[0]; ot[1] += o[1]; ot[2] += o[2]; ot[3] += o[3];
      lt += red_l[slot * SG + i];
    }
  }
  if (!valid) return;
  const int node = r / a.G, head = g * a.G + (r - node * a.G);
  uint16_t* out = (uint16_t*)a.out + (((size_t)b * a.D + node) * a.Hq + head) * DH + 4 * lane;
  const size_t li = ((size_t)b * a.D + node) * a.Hq + head;
  if (st != TV_SEQ_OK) {
    *(uint2*)out = make_uint2(0u, 0u);
    if (a.lse != nullptr && lane == 0) a.lse[li] = -INFINITY;
    return;
  }
  const float inv = 1.0f / lt;
  uint2 pk;
  pk.x = (uint32_t)f32_to_bf16_bits(ot[0] * inv) | ((uint32_t)f32_to_bf16_bits(ot[1] * inv) << 16);
  pk.y = (uint32_t)f32_to_bf16_bits(ot[2] * inv) | ((uint32_t)f32_to_bf16_bits(ot[3] * inv) << 16);
  *(uint2*)out = pk;
  if (a.lse != nullptr && lane == 0) a.lse[li] = (M + log2f(lt)) * kLn2;
}

template <int SG, int JR>
static hipError_t launch_merge_t(const AttnArgs& a, hipStream_t s) {
  const dim3 grid(a.Hkv * a.row_blocks * (a.unit_rows / (8 / SG)), a.B);
  if (a.nt_partials) hipLaunchKernelGGL((k_attn_merge<SG, JR, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_attn_merge<SG, JR, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// slices per unit at most n_max: the fewest groups per row that keep a thread at <= 4 loads
// (up to 32 slices), then more loads per thread
static hipError_t launch_merge(const AttnArgs& a, hipStream_t s) {
  const int n = a.merge_nmax;
  if (n <= 4) return launch_merge_t<1, 4>(a, s);
  if (n <= 8) return launch_merge_t<2, 4>(a, s);
  if (n <= 16) return launch_merge_t<4, 4>(a, s);
  if (n <= 32) return launch_merge_t<8, 4>(a, s);
  if (n <= 64) return launch_merge_t<8, 8>(a, s);
  return launch_merge_t<8, 16>(a, s);
}

template <typename T, int DH, bool NT>
static hipError_t launch_finish_nt(const AttnArgs& a, hipStream_t s) {
  const size_t lds = a.fused_tree ? 0 : (size_t)a.D * DH * sizeof(T) * 2;
  if (lds > 65536) {  // beyond the default dynamic-LDS limit (fp32, d = 128, D > 32)
    hipError_t e = hipFuncSetAttribute((const void*)k_attn_finish<T, DH, NT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.Hkv * a.row_blocks * (a.unit_rows / kFinishWaves), a.B), block(kFinishWaves * 64);
  hipLaunchKernelGGL((k_attn_finish<T, DH, NT>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_finish_t(const AttnArgs& a, hipStream_t s) {
  return a.nt_partials ? launch_finish_nt<T, DH, true>(a, s) : launch_finish_nt<T, DH, false>(a, s);
}

hipError_t launch_attn_finish(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.fused_tree) return launch_merge(a, s);  // (the MFMA path: bf16, d = 128)
  if (a.dtype == TV_BF16) return a.d == 128 ? launch_finish_t<uint16_t, 128>(a, s) : launch_finish_t<uint16_t, 64>(a, s);
  return a.d == 128 ? launch_finish_t<float, 128>(a, s) : launch_finish_t<float, 64>(a, s);
}

}  // namespace tv
