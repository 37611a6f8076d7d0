// Draft-tree construction on the device: expansion of the top-k tokens of each expanded
// node's draft logits, cumulative log-softmax scores, pruning to the verification budget.
// TSD-V4 §2.1 (the draft expands a candidate tree; pruning keeps promising candidates so
// that the verified tokens stay within the budget), §4.1 (draft extend organises the
// candidate topology) and §4.3 (such metadata can be prepared on the device, so the host
// does not sit between the draft model and verification).
//
// Node e (the root is 0) is expanded into candidates e*k + 1 .. e*k + k: the k tokens
// with the largest logits of row e (ties: the smaller token id), in that order; nodes of
// depth < steps are expanded, so there are E = 1 + k + ... + k^(steps-1) rows and
// N = k + ... + k^steps candidates.  A candidate's score is its parent's plus
// log_softmax(row of the parent)[token] (the root's is 0); the D - 1 best candidates are
// kept (ties: shallower, then smaller creation index) and numbered 1 .. D-1 by rank.
// Scores are kept in float64, so the ranking (an integer result) is not at the mercy of
// float32 rounding.
//
// One workgroup of 512 threads per sequence.  Each wave takes rows e = wave, wave + 8,
// ...: the row max (wave max), the normaliser sum exp(x - max) in float64 (wave sum), and
// the top k as k successive wave argmaxes, pick r taking the best token strictly after
// pick r-1 in the (logit desc, id asc) order, so no chosen set is kept.  A vocabulary of
// up to 1024 is read once into registers (16 values per lane) for all of these passes.  Then the scores
// are accumulated level by level in LDS, each candidate's rank is the number of
// candidates that beat it, and the kept ones are written out.
#include "tv_launch.h"

namespace tv {

namespace {
constexpr int kDtThreads = 512;
constexpr int kVpl = 16;  // vocabulary entries a lane keeps in registers (vocab <= 1024)

// (v, t) comes before (bv, bt) in the order logits descending, ids ascending
__device__ __forceinline__ bool before(float v, int t, float bv, int bt) {
  return v > bv || (v == bv && t < bt);
}
}  // namespace

__global__ __launch_bounds__(kDtThreads) void k_draft_tree(int k, int steps, int D, int V, int E, int N,
                                                           const float* __restrict__ logits,
                                                           const int32_t* __restrict__ root_tok,
                                                           int32_t* __restrict__ parents,
                                                           int32_t* __restrict__ draft_tok, float* __restrict__ cum_out) {
  __shared__ double score_s[TV_DT_MAX_CAND + 1];  // log-softmax increment, then cumulative score
  __shared__ int tok_s[TV_DT_MAX_CAND + 1];
  __shared__ int slot_s[TV_DT_MAX_CAND + 1];      // output node of a kept candidate, else -1
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* lg = logits + (size_t)b * E * V;

  // 1. per expanded row: normaliser and top k
  const bool cached = V <= 64 * kVpl;  // uniform
  for (int e = w; e < E; e += kDtThreads / 64) {
    const float* row = lg + (size_t)e * V;
    float xv[kVpl];
    float m = -INFINITY;
    if (cached) {
#pragma unroll
      for (int i = 0; i < kVpl; ++i) {
        const int t = lane + 64 * i;
        xv[i] = t < V ? row[t] : -INFINITY;
        m = fmaxf(m, xv[i]);
      }
    } else {
      for (int t = lane; t < V; t += 64) m = fmaxf(m, row[t]);
    }
    m = wave_max(m);
    double s = 0.0;
    if (m != -INFINITY) {
      if (cached) {
#pragma unroll
        for (int i = 0; i < kVpl; ++i)
          if (lane + 64 * i < V) s += exp((double)xv[i] - (double)m);
      } else {
        for (int t = lane; t < V; t += 64) s += exp((double)row[t] - (double)m);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    const double lse = m == -INFINITY ? -INFINITY : (double)m + log(s);
    float pv = INFINITY;  // previous pick: (pv, pt); every token comes after (+inf, -1)
    int pt = -1;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bt = 0x7fffffff;
      if (cached) {
#pragma unroll
        for (int i = 0; i < kVpl; ++i) {
          const int t = lane + 64 * i;
          if (t < V && before(pv, pt, xv[i], t) && before(xv[i], t, bv, bt)) {
            bv = xv[i];
            bt = t;
          }
        }
      } else {
        for (int t = lane; t < V; t += 64) {
          const float v = row[t];
          if (before(pv, pt, v, t) && before(v, t, bv, bt)) {
            bv = v;
            bt = t;
          }
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int ot = __shfl_xor(bt, o, 64);
        if (before(ov, ot, bv, bt)) {
          bv = ov;
          bt = ot;
        }
      }
      if (lane == 0) {
        const int c = e * k + r + 1;
        tok_s[c] = bt;
        score_s[c] = lse == -INFINITY ? -INFINITY : (double)bv - lse;
      }
      pv = bv;
      pt = bt;
    }
  }
  if (tid == 0) score_s[0] = 0.0;
  __syncthreads();

  // 2. cumulative scores, one level at a time (a level's parents are the level above)
  int lo = 1, width = k;
  for (int l = 1; l <= steps; ++l) {
    for (int c = lo + tid; c < lo + width; c += kDtThreads) score_s[c] += score_s[(c - 1) / k];
    __syncthreads();
    lo += width;
    width *= k;
  }

  // 3. rank of every candidate; the best D - 1 get output nodes 1 .. D-1
  for (int c = 1 + tid; c <= N; c += kDtThreads) {
    const double sc = score_s[c];
    // depth of c: the level whose index range holds it
    int dc = 1;
    for (int lo2 = 1, w2 = k; c >= lo2 + w2; lo2 += w2, w2 *= k) ++dc;
    int rank = 0;
    int lo3 = 1, w3 = k, d3 = 1;
    for (int c2 = 1; c2 <= N; ++c2) {
      if (c2 == lo3 + w3) {
        lo3 += w3;
        w3 *= k;
        ++d3;
      }
      const double s2 = score_s[c2];
      rank += (s2 > sc || (s2 == sc && (d3 < dc || (d3 == dc && c2 < c)))) ? 1 : 0;
    }
    slot_s[c] = rank < D - 1 ? rank + 1 : -1;
  }
  if (tid == 0) slot_s[0] = 0;
  __syncthreads();

  // 4. the tree: root, then the kept candidates in rank order
  int32_t* par = parents + (size_t)b * D;
  int32_t* dt = draft_tok + (size_t)b * D;
  float* co = cum_out != nullptr ? cum_out + (size_t)b * D : nullptr;
  if (tid == 0) {
    par[0] = -1;
    dt[0] = root_tok[b];
    if (co != nullptr) co[0] = 0.f;
  }
  for (int c = 1 + tid; c <= N; c += kDtThreads) {
    const int slot = slot_s[c];
    if (slot < 0) continue;
    par[slot] = slot_s[(c - 1) / k];  // a parent always outranks its children
    dt[slot] = tok_s[c];
    if (co != nullptr) co[slot] = (float)score_s[c];
  }
}

hipError_t launch_draft_tree(int B, int k, int steps, int D, int V, int E, int N, const float* logits,
                             const int32_t* root_tok, int32_t* parents, int32_t* draft_tok, float* cum,
                             hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_draft_tree, dim3(B), dim3(kDtThreads), 0, s, k, steps, D, V, E, N, logits, root_tok,
                     parents, draft_tok, cum);
  return hipGetLastError();
}

}  // namespace tv
