// Host-side launchers of the library's kernels (one per kernel file); the C entry points
// in tv_host.cpp validate arguments and call these.
#pragma once
#include "tv_common.h"

namespace tv {

hipError_t launch_tree_mask(int B, int D, const int32_t* parents, uint64_t* anc, int32_t* depth,
                            int32_t* seq_err, hipStream_t s);
hipError_t launch_accept(int B, int D, const int32_t* parents, const uint64_t* anc,
                         const int32_t* depth, const int32_t* draft, const int32_t* target,
                         const int32_t* seq_err, int32_t* m, int32_t* path, int32_t* bonus,
                         hipStream_t s);
hipError_t launch_refresh(int D, const tv_state& st, const tv_scratch& sc, const void* k_tree,
                          const void* v_tree, const int32_t* m, const int32_t* path,
                          int32_t* commit_log, int32_t* seq_err, hipStream_t s);
hipError_t launch_accept_refresh(int D, const tv_state& st, const tv_scratch& sc, const int32_t* parents,
                                 const uint64_t* anc, const int32_t* depth, const int32_t* draft,
                                 const int32_t* target, const void* k_tree, const void* v_tree, int32_t* m,
                                 int32_t* path, int32_t* bonus, int32_t* commit_log, int32_t* seq_err,
                                 hipStream_t s);
hipError_t launch_compress(const tv_state& st, const void* raw_k, const void* raw_v, int max_len,
                           int32_t* seq_err, hipStream_t s);
hipError_t launch_attn_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_valu(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_finish(const AttnArgs& a, hipStream_t s);
hipError_t launch_scratch(const AttnArgs& a, hipStream_t s);
hipError_t launch_draft_tree(int B, int k, int steps, int D, int V, int E, int N, const float* logits,
                             const int32_t* root_tok, int32_t* parents, int32_t* draft_tok, float* cum,
                             hipStream_t s);

}  // namespace tv
