/*
 * tv.h — C ABI of the target-verify path of tree-structured speculative decoding
 * over sequence-compressed attention KV, for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "Adapting Tree-Structured Speculative Decoding to
 * DeepSeek-V4 for Efficient Inference" (cited TSD-V4; that page has no numbered
 * headings, section numbers are inferred from its own "Sec. 5.2/5.3" references
 * and the order of its topics).  One decoding step of the path is:
 *
 *   tv_build_tree_mask   verify preprocess: tree -> verification plan      (§4.1)
 *   tv_verify_attn       branch-aware causal attention + per-chain scratch  (§3.1, §4.1, §4.2)
 *   tv_accept            accepted-path selection                            (§3.1, §4.4)
 *   tv_refresh_state     accepted-path refresh of the compressed state      (§3.2, §4.2, §4.3)
 *   tv_accept_refresh    the two calls above in one launch                  (§4.3)
 *
 * plus tv_compress_prefix, which builds the compressed state of a raw prefix.
 *
 * Conventions
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or keeps a pointer after a call returns.  The
 *    tv_state / tv_scratch structs themselves are host structs passed by address;
 *    they are read during the call only.  Arrays of elements or fp32 sums (Q, tree
 *    K/V, pools, open sums, tails, scratch, the output, the workspace) must be
 *    16-byte aligned: the kernels move them in 8- and 16-byte pieces.
 *  - Every call is asynchronous on `stream`; none synchronises the device or
 *    allocates, so the four-call step can be captured in a hipGraph.
 *  - Host-checkable argument errors return TV_EINVAL / TV_EUNSUPPORTED /
 *    TV_EWORKSPACE before anything is launched (device memory untouched);
 *    tv_last_error() then describes the problem.  Launch failures return TV_EHIP.
 *  - Data-dependent errors are per sequence, in seq_err[b] (TV_SEQ_*): a
 *    sequence with a nonzero code is skipped by every later call of the step and
 *    its persistent state is left unchanged.
 *  - D counts the tree's root.  Node 0 is the root: the last committed token,
 *    whose K/V is computed by this verify and is not yet in the state.  Nodes are
 *    in topological order: parents[0] = -1 and 0 <= parents[i] < i.  D <= 64.
 *  - A node's position is P + depth(node), P = committed length of its sequence.
 *  - Element types: TV_BF16 (bfloat16) or TV_F32, the same for Q, tree K/V, pools,
 *    tail, scratch entries and the attention output.  Open-block sums, the LSE and
 *    all accumulation are fp32.
 *  - Compression stand-in (the pages leave CSA/HCA's compressor undefined): level
 *    l with block size C keeps one entry per complete aligned block [jC, jC+C) of
 *    committed positions, the unweighted mean of its K (and of its V) per KV head.
 */
#ifndef TV_H
#define TV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define TV_API __attribute__((visibility("default")))
#else
#define TV_API
#endif

#define TV_VERSION 140      /* 1.4.0: tv_scratch.deferred (levels brought up to date by the refresh) */
#define TV_MAX_LEVELS 2
#define TV_MAX_D 64
#define TV_TILE_RUN 16     /* tiles of one (sequence, KV head) kept together in a contiguous pool */
#define TV_POOL_ALIGN 64    /* every pool capacity must be a multiple of this */
#define TV_DT_MAX_CAND 2048 /* candidates of an expanded draft tree (tv_build_draft_tree) */

typedef enum {
  TV_OK = 0,
  TV_EINVAL = -1,        /* bad argument (null pointer, size out of range, ...) */
  TV_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. head dim other than 64/128) */
  TV_EWORKSPACE = -3,    /* workspace smaller than tv_verify_attn_workspace_bytes() */
  TV_EHIP = -4           /* a HIP launch failed */
} tv_status;

typedef enum { TV_F32 = 0, TV_BF16 = 1 } tv_dtype;

/* seq_err codes (int32, one per sequence) */
enum {
  TV_SEQ_OK = 0,
  TV_SEQ_BAD_PARENT = 1,  /* parents[b] is not a topologically ordered tree */
  TV_SEQ_POOL_FULL = 2,   /* committing would exceed a pool's capacity */
  TV_SEQ_BAD_PREFIX = 3,  /* tv_compress_prefix: P[b] outside [0, max_len] */
  TV_SEQ_BAD_PATH = 4,    /* tv_refresh_state: m or a path node out of range, or P < 0 */
  TV_SEQ_BAD_PAGE = 5     /* a page-table entry needed for a write is outside [0, num_pages) */
};

/* One compression level (the pages' C4 / C128 compressed states, TSD-V4 §2.2, §4.3).
 * A level's entries live in 64-entry tiles (TV_POOL_ALIGN): tile t of (sequence b, KV
 * head g) holds entries 64t .. 64t+63, as 64 rows of d (K) and as d rows of 64 (V,
 * transposed inside the tile).  Contiguous pool (page_table == NULL), T = cap/64 tiles per
 * (b, g), R = TV_TILE_RUN: for q < floor(T/R), tiles R*q .. R*q+R-1 of (b, g) are tiles
 * ((q*B + b)*Hkv + g)*R + 0 .. R-1 of k and vt; the last T mod R tiles of (b, g) are tiles
 * floor(T/R)*B*Hkv*R + (b*Hkv + g)*(T mod R) + 0 ..  (k: [B*Hkv*T][64][d] tiles, vt:
 * [B*Hkv*T][d][64]).  A step reads every sequence's prefix at once; this keeps those reads
 * within one window of memory instead of at a fixed stride of one sequence's pool.  The
 * addresses depend on B, so a contiguous pool serves a fixed number of sequence slots; a
 * batch that grows and shrinks uses the paged form.
 * Paged pool (TSD-V4 §4.2: a page-based pool whose pages are referenced by pointers):
 * k and vt hold num_pages physical pages, each
 * the tiles of all Hkv heads for 64 entries ([num_pages][Hkv][64][d] and
 * [num_pages][Hkv][d][64]); page_table[b][t] is the physical page of sequence b's
 * entries 64t .. 64t+63, and cap = 64 * pages_per_seq.  Page ids outside
 * [0, num_pages) are never dereferenced: attention reads zeros for them, refresh and
 * compression flag the sequence TV_SEQ_BAD_PAGE. */
typedef struct {
  int32_t C;        /* block size: tokens per compressed entry (>= 1) */
  int32_t cap;      /* capacity in entries, a multiple of TV_POOL_ALIGN */
  void* k;          /* contiguous: B*Hkv*cap/64 tiles [64][d] (see above); paged: [num_pages][Hkv][64][d] */
  void* vt;         /* contiguous: B*Hkv*cap/64 tiles [d][64]; paged: [num_pages][Hkv][d][64] */
  int32_t* n;       /* [B] committed entries of each sequence (kept equal to P/C) */
  float* open_k;    /* [B][Hkv][d] fp32 sum of the committed tokens of the open block */
  float* open_v;    /* [B][Hkv][d] */
  int32_t* page_table;     /* [B][pages_per_seq], or NULL for a contiguous pool */
  int32_t pages_per_seq;   /* paged: cap / 64 */
  int32_t num_pages;       /* paged: physical pages in k and vt */
} tv_level;

/* Persistent compressed state of B sequences (TSD-V4 §4.2 "persistent context"). */
typedef struct {
  int32_t B, Hkv, d;
  int32_t dtype;                /* tv_dtype */
  int32_t n_levels;             /* 0..TV_MAX_LEVELS, finest (smallest C) first, C strictly increasing */
  tv_level lvl[TV_MAX_LEVELS];
  void* tail_k;                 /* [B][Hkv][lvl[0].C-1][d] raw tokens of the finest level's open */
  void* tail_v;                 /*   block: positions floor(P/C0)*C0 .. P-1 (may be NULL if C0 == 1) */
  int32_t* P;                   /* [B] committed length */
} tv_state;

/* Per-branch temporary compression results (TSD-V4 §4.2 scratch pad), per level l:
 * entry for node i is valid only if node i closes a block of that level, i.e.
 * (P + depth(i) + 1) % C == 0; open sums are the open block after node i along
 * its own chain (zero where it closes).  Overwritten by every tv_verify_attn.
 *
 * in_place (optional; TSD-V4 §4.3: with a single candidate chain, or when the accepted
 * chain is the one already cached, the refresh can be skipped): when non-NULL,
 * tv_verify_attn also writes the entries that the nodes of one chain close straight into
 * their pool slots -- the chain ending at the deepest node, smallest index among equals
 * (the path full acceptance selects; the whole tree when it is a single chain) -- and sets
 * in_place[b] to that chain's node mask (0 for a flagged sequence).  Those slots lie at
 * or beyond the committed counts, so the committed state does not change, and only slots
 * below the capacity whose page exists are written.  tv_refresh_state / tv_accept_refresh
 * given the same struct then copy only the committed entries of nodes outside the mask.
 * The resulting state is bit-identical to the one without in_place, apart from pool
 * slots at or beyond the new counts (never read).
 *
 * deferred (TSD-V4 §4.3: C4 and C128 have different refresh schedules; the coarse level is
 * compressed rarely, so its cache writes can be delayed and combined once the accepted
 * path is known): bit l set = level l gets no scratch states.  tv_verify_attn builds none
 * for it (its four pointers may be NULL) and writes none of its entries in place;
 * tv_refresh_state / tv_accept_refresh then bring that level up to date from the accepted
 * path's own tokens in one pass: the committed open sum plus the path tokens in path
 * order in fp32, each block the path closes written once as sum / C (one rounding), the
 * rest left as the new open sum.  The additions and roundings are those the scratch pad
 * makes along the same chain, so the state is bit-identical to the one without deferral.
 * Bits at or beyond n_levels are invalid (TV_EINVAL). */
typedef struct {
  void* entry_k[TV_MAX_LEVELS];   /* [B][D][Hkv][d] element dtype */
  void* entry_v[TV_MAX_LEVELS];   /* [B][D][Hkv][d] */
  float* open_k[TV_MAX_LEVELS];   /* [B][D][Hkv][d] fp32 */
  float* open_v[TV_MAX_LEVELS];   /* [B][D][Hkv][d] */
  uint64_t* in_place;             /* [B] out of tv_verify_attn, in to the refresh; NULL = off */
  uint32_t deferred;              /* levels updated from the accepted path by the refresh (bit l) */
} tv_scratch;

/*
 * Verify preprocess (TSD-V4 §4.1: the tree becomes a verification plan describing
 * the candidate chains and their compression boundaries; §4.3: this metadata is
 * prepared on the device).
 *   parents  [B][D] int32 in
 *   anc      [B][D] uint64 out: bit j of anc[b][i] set iff node j is an ancestor of
 *            node i or i itself (the chain of node i)
 *   depth    [B][D] int32 out: depth(i), root = 0
 *   seq_err  [B] int32 out: TV_SEQ_OK, or TV_SEQ_BAD_PARENT (then anc = depth = 0)
 * B >= 0 (B == 0 is a no-op), 1 <= D <= 64.
 */
TV_API tv_status tv_build_tree_mask(int B, int D, const int32_t* parents, uint64_t* anc,
                                    int32_t* depth, int32_t* seq_err, hipStream_t stream);

/*
 * Draft-tree construction (TSD-V4 §2.1: the draft expands the accepted prefix into a
 * candidate tree, and pruning keeps promising candidates within the verification-token
 * budget; §4.1 draft extend; §4.3 such metadata prepared on the device).  Expansion:
 * node e (root = 0, then candidates in creation order) gets the topk tokens with the
 * largest logits of its row (ties: smaller token id) as children e*topk + 1 ..
 * e*topk + topk, for `steps` levels, so E = 1 + topk + ... + topk^(steps-1) nodes are
 * expanded and N = topk + ... + topk^steps candidates created.  A candidate's score is
 * its parent's plus log_softmax(parent's row)[token] (root: 0), computed in float64.
 * Pruning keeps the D - 1 best candidates (ties: shallower, then earlier created);
 * the tree is the root followed by them in rank order, so 0 <= parents[i] < i.
 *   logits    [B][E][vocab] fp32 in: row e = draft logits after node e (finite or -inf,
 *             at least one finite value per row)
 *   root_tok  [B] in: the root's token (the last committed token)
 *   parents   [B][D] out (parents[b][0] = -1), draft_tok [B][D] out
 *   cum_logp  [B][D] fp32 out, each node's score (NULL = not wanted)
 * Limits: topk >= 1, steps >= 1, vocab >= topk, N <= TV_DT_MAX_CAND,
 * 1 <= D <= min(TV_MAX_D, N + 1).  The output feeds tv_build_tree_mask directly.
 */
TV_API tv_status tv_build_draft_tree(int B, int topk, int steps, int D, int vocab, const float* logits,
                                     const int32_t* root_tok, int32_t* parents, int32_t* draft_tok,
                                     float* cum_logp, hipStream_t stream);

/*
 * Bytes of device workspace tv_verify_attn needs for this state shape when the
 * shared-prefix stream is cut into num_parts slices of equal length to within one
 * 64-entry chunk, one workgroup each (0 = the library's choice for the current device:
 * one full round of resident workgroups, at least 4 chunks each, as a multiple of the
 * prefix count where that keeps 7/8 of them, and one per compute unit for streams of 16
 * to 32 chunks per unit; the same value must then be passed to tv_verify_attn).  The slices run
 * over every (sequence, KV head, block of query rows) prefix laid end to end, so any
 * batch size keeps the whole GPU busy; a prefix split over several slices gets one
 * partial (max, sum, unnormalised output) per slice, merged after the stream.  When no
 * prefix is split (e.g. 64 sequences of 8 KV heads on 256 compute units) nothing is
 * written to the workspace and 256 bytes are asked for.  The contents need no
 * initialisation and are dead after the call.  Returns 0 on invalid arguments.
 */
TV_API size_t tv_verify_attn_workspace_bytes(int D, int Hq, const tv_state* st, int num_parts);

/*
 * Branch-aware causal verification (TSD-V4 §3.1: each candidate attends to the
 * accepted context and to the ancestors on its own branch only; §4.1 target
 * verify) plus chain-wise compression into the scratch pad (§4.1: branches are
 * compressed independently after they diverge; §4.2: temporary states stay in
 * the scratch pad until acceptance).
 *
 * For node i, query head h (KV head g = h / (Hq/Hkv)) the visible rows are: every
 * committed entry of every level (n[l][b] of them), the finest level's tail
 * (P mod C0 raw tokens), and the tree nodes j with bit j of anc[b][i] set.  One
 * softmax over all of them with scale 1/sqrt(d); rows not visible are never read.
 *   q        [B][D][Hq][d]  in      k_tree, v_tree [B][D][Hkv][d] in
 *   anc, depth from tv_build_tree_mask; seq_err [B] in (NULL = all OK)
 *   scratch  out (NULL = do not build it); out [B][D][Hq][d] out (element dtype)
 *   lse      [B][D][Hq] fp32 out, natural-log softmax normaliser (NULL = not wanted)
 *   workspace: >= tv_verify_attn_workspace_bytes(D, Hq, st, num_parts) bytes, 16-byte aligned
 * Supported: d in {64, 128}; Hq % Hkv == 0; TV_BF16 with d = 128 runs the MFMA
 * kernel, everything else the fp32 vector kernel.
 */
TV_API tv_status tv_verify_attn(int D, int Hq, const void* q, const void* k_tree,
                                const void* v_tree, const uint64_t* anc, const int32_t* depth,
                                const int32_t* seq_err, const tv_state* st,
                                const tv_scratch* scratch, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, int num_parts,
                                hipStream_t stream);

/*
 * tv_verify_attn for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results as tv_verify_attn (the same kernels, bit-identical outputs and scratch pad),
 * without workspace / workspace_bytes: the split-prefix partials go to a device array
 * of TV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on until the
 * process ends (its address is looked up on the first call on each device; nothing is
 * allocated by any call).  A shape whose partials need more (tv_verify_attn_workspace_bytes
 * > TV_NOALLOC_SCRATCH_BYTES, i.e. many prefixes split over many slices) returns
 * TV_EWORKSPACE before any launch.  The array needs no clearing: each call writes every
 * partial it reads.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (two streams, two threads) race and give undefined results; calls
 * ordered on one stream are safe.
 */
#define TV_NOALLOC_SCRATCH_BYTES (24u << 20)
TV_API tv_status tv_verify_attn_noalloc(int D, int Hq, const void* q, const void* k_tree,
                                        const void* v_tree, const uint64_t* anc, const int32_t* depth,
                                        const int32_t* seq_err, const tv_state* st,
                                        const tv_scratch* scratch, void* out, float* lse, int num_parts,
                                        hipStream_t stream);

/*
 * Branch-aware attention of one draft-decode level (TSD-V4 §4.1: draft decode computes
 * the candidates' representations under the tree topology; §4.3: the same metadata
 * serves draft and verify).  The candidate tree grows level by level in creation order
 * (parents before children), so the nodes created so far are the first D nodes and
 * their plan is the first D entries of each row of the whole expansion's plan: anc is
 * [B][anc_ld] from one tv_build_tree_mask call over all anc_ld nodes, shared by every
 * level.  Rows are computed for all D nodes with the same visibility as
 * tv_verify_attn (no scratch pad); a node's row depends only on its own chain, so the
 * rows of earlier levels are what those levels produced.
 *   q [B][D][Hq][d], k_tree, v_tree [B][D][Hkv][d], out [B][D][Hq][d], lse [B][D][Hq]
 *   workspace: >= tv_verify_attn_workspace_bytes(D, Hq, st, num_parts) bytes
 * 1 <= D <= anc_ld <= TV_MAX_D.
 */
TV_API tv_status tv_draft_attn(int D, int anc_ld, int Hq, const void* q, const void* k_tree,
                               const void* v_tree, const uint64_t* anc, const int32_t* seq_err,
                               const tv_state* st, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, int num_parts, hipStream_t stream);

/*
 * Accepted-path selection (TSD-V4 §3.1: the result is a specific path through the
 * tree; §4.4 accepted-path selection).  Greedy rule: draft node i >= 1 is correct
 * iff draft_tok[i] == target_tok[parent(i)] (target_tok[u] = the target model's
 * greedy token after node u); a node is accepted iff every node of its chain below
 * the root is correct.  The path ends at the deepest accepted node, smallest index
 * among equals.
 *   m      [B] out: accepted draft tokens (= depth of the path's last node)
 *   path   [B][D] out: path nodes root first, -1 after index m
 *   bonus  [B] out: target_tok of the path's last node (the next step's root)
 * Sequences with seq_err != 0 get m = -1, path = -1, bonus = -1.
 */
TV_API tv_status tv_accept(int B, int D, const int32_t* parents, const uint64_t* anc,
                           const int32_t* depth, const int32_t* draft_tok,
                           const int32_t* target_tok, const int32_t* seq_err, int32_t* m,
                           int32_t* path, int32_t* bonus, hipStream_t stream);

/*
 * Accepted-path refresh (TSD-V4 §3.2: token history, cache and compressed states
 * must describe the same prefix; §4.2: only the accepted path's states update the
 * persistent state, rejected branches are dropped; §4.3 C4/C128 state updates).
 * The root and path[1..m] become committed tokens at positions P..P+m; P' = P+m+1.
 * For each level, every block j with floor(P/C) <= j < floor(P'/C) takes the
 * scratch entry of the path node at its last position; the open sums become the
 * path leaf's scratch open sums; the tail becomes positions floor(P'/C0)*C0..P'-1.
 *   st: updated in place (pools, n, open sums, tail, P)
 *   commit_log [B][n_levels][D][2] int32 out: rows (destination slot, source node),
 *              -1 padded (NULL = not wanted)
 *   seq_err [B] in/out: skipped if nonzero; set to TV_SEQ_POOL_FULL (state untouched)
 *              if a level would exceed its capacity, TV_SEQ_BAD_PATH if m >= D or a
 *              path node is outside 0..D-1 (state untouched)
 * "State untouched" means P, the counts, open sums, tail and every committed pool slot;
 * with scratch->in_place the verify may already have written slots at or beyond the
 * committed counts, which nothing reads until a later refresh commits them.
 */
TV_API tv_status tv_refresh_state(int D, const tv_state* st, const tv_scratch* scratch,
                                  const void* k_tree, const void* v_tree, const int32_t* m,
                                  const int32_t* path, int32_t* commit_log, int32_t* seq_err,
                                  hipStream_t stream);

/*
 * tv_accept followed by tv_refresh_state in one launch (TSD-V4 §4.3: keeping the
 * refresh cheap; on this path its cost is launch and round-trip latency, not bytes).
 * One workgroup per sequence: its first wave selects the accepted path into on-chip
 * memory and the workgroup refreshes from it, so m and the path are not read back.
 * Arguments as for the two calls (B = st->B); m, path and bonus are written as
 * tv_accept writes them, the state, commit_log and seq_err as tv_refresh_state does.
 * Results are identical to the two calls made in order.
 */
TV_API tv_status tv_accept_refresh(int D, const tv_state* st, const tv_scratch* scratch,
                                   const int32_t* parents, const uint64_t* anc, const int32_t* depth,
                                   const int32_t* draft_tok, const int32_t* target_tok,
                                   const void* k_tree, const void* v_tree, int32_t* m, int32_t* path,
                                   int32_t* bonus, int32_t* commit_log, int32_t* seq_err,
                                   hipStream_t stream);

/*
 * Compressed state of a raw committed prefix (TSD-V4 §2.2: compression along the
 * sequence axis at several granularities).  Reads P[b] (set by the caller) and
 * the raw tokens raw_k/raw_v [B][Hkv][max_len][d]; writes every level's entries
 * 0..P/C-1, n = P/C, open sums and the tail.  seq_err[b] [B] out: TV_SEQ_OK,
 * TV_SEQ_BAD_PREFIX (P outside [0, max_len]) or TV_SEQ_POOL_FULL.
 */
TV_API tv_status tv_compress_prefix(const tv_state* st, const void* raw_k, const void* raw_v,
                                    int max_len, int32_t* seq_err, hipStream_t stream);

TV_API const char* tv_status_string(tv_status s);
TV_API const char* tv_last_error(void);   /* this thread's last argument/launch error */
TV_API int tv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TV_H */
