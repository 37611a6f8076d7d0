// libtv host entry points: argument validation, split-KV planning and kernel
// launches.  Nothing here allocates device memory or synchronises; every check
// that can be made on the host happens before the first launch of a call.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "tv.h"
#include "tv_launch.h"

namespace {

thread_local char g_err[512] = "";

tv_status fail(tv_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

tv_status ok() {
  g_err[0] = '\0';
  return TV_OK;
}

tv_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TV_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape and pointer checks of a state; `need_tail` only matters when a level exists.
tv_status check_state(const tv_state* st) {
  if (st == nullptr) return fail(TV_EINVAL, "state is NULL");
  if (st->B < 0) return fail(TV_EINVAL, "B = %d < 0", st->B);
  if (st->Hkv < 1) return fail(TV_EINVAL, "Hkv = %d < 1", st->Hkv);
  if (st->d != 64 && st->d != 128) return fail(TV_EUNSUPPORTED, "head dim %d (supported: 64, 128)", st->d);
  if (st->dtype != TV_F32 && st->dtype != TV_BF16) return fail(TV_EINVAL, "dtype %d", st->dtype);
  if (st->n_levels < 0 || st->n_levels > TV_MAX_LEVELS)
    return fail(TV_EINVAL, "n_levels = %d (0..%d)", st->n_levels, TV_MAX_LEVELS);
  if (st->P == nullptr) return fail(TV_EINVAL, "state P is NULL");
  for (int l = 0; l < st->n_levels; ++l) {
    const tv_level& L = st->lvl[l];
    if (L.C < 1) return fail(TV_EINVAL, "level %d: C = %d < 1", l, L.C);
    if (l > 0 && L.C <= st->lvl[l - 1].C) return fail(TV_EINVAL, "level block sizes must increase");
    if (L.cap < 0 || L.cap % TV_POOL_ALIGN != 0)
      return fail(TV_EINVAL, "level %d: cap = %d must be a non-negative multiple of %d", l, L.cap,
                  TV_POOL_ALIGN);
    if (!L.k || !L.vt || !L.n || !L.open_k || !L.open_v)
      return fail(TV_EINVAL, "level %d: NULL pool/count/open-sum pointer", l);
    if (!aligned16(L.k) || !aligned16(L.vt) || !aligned16(L.open_k) || !aligned16(L.open_v))
      return fail(TV_EINVAL, "level %d: pools and open sums must be 16-byte aligned", l);
    if (L.page_table != nullptr) {
      if (L.pages_per_seq < 0 || (long long)L.pages_per_seq * TV_POOL_ALIGN != L.cap)
        return fail(TV_EINVAL, "level %d: paged pool needs cap = %d * pages_per_seq", l, TV_POOL_ALIGN);
      if (L.num_pages < 1) return fail(TV_EINVAL, "level %d: num_pages = %d < 1", l, L.num_pages);
    }
  }
  for (int l = 1; l < st->n_levels; ++l)
    if ((st->lvl[l].page_table == nullptr) != (st->lvl[0].page_table == nullptr))
      return fail(TV_EINVAL, "either every level is paged or none is");
  if (st->n_levels > 0 && st->lvl[0].C > 1 && (!st->tail_k || !st->tail_v))
    return fail(TV_EINVAL, "tail pointers are NULL");
  if (!aligned16(st->tail_k) || !aligned16(st->tail_v)) return fail(TV_EINVAL, "tails must be 16-byte aligned");
  return ok();
}

// Levels marked deferred must exist.
tv_status check_deferred(const tv_scratch* sc, const tv_state* st) {
  if ((sc->deferred >> st->n_levels) != 0u)
    return fail(TV_EINVAL, "scratch.deferred = 0x%x marks levels beyond n_levels = %d", sc->deferred, st->n_levels);
  return ok();
}

// compute units of the current device (asked once per device)
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices && (cus = cached[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The device memory behind tv_verify_attn_noalloc: one copy of this array on every GPU
// the library runs on, held until the process ends.  In host code the name `scratch` is a
// host-side stand-in, not a device address: each device's address is looked up once
// (hipGetSymbolAddress, with that device current) and only that address is ever used.
static __device__ __attribute__((aligned(256))) unsigned char scratch[TV_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device (looked up on the first call there).
tv_status noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> cached[kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TV_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(mu);
    p = cached[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(TV_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      cached[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ok();
}

struct Plan {
  bool mfma;        // bf16 with d = 128 runs the MFMA prefix kernel, everything else the vector kernel
  bool fused_tree;  // the MFMA kernel attends to the raw tail and the tree chunk itself
  int tree_tiles;   // 16-entry tiles of that chunk
  int R, unit_rows, row_blocks, tmax, parts;
  long long per_lo;  // chunks per slice, rounded down
  long long units;
  bool too_big;     // units * tmax chunk slots do not fit the kernels' 32-bit indices
  bool nt_partials; // partials are written and read with the nontemporal hint
  bool all_whole;   // every unit is one workgroup's and the prefix kernel writes the rows: no partials
  size_t ws_o_bytes, ws_ml_off, total;
  bool fold;        // the MFMA prefix launch has room for the scratch pad's B*D workgroups ahead of the stream
  bool pad_after;   // else they follow the stream's workgroups in the same launch
};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Prefix-stream partition (see AttnArgs).  Auto mode runs one round of persistent
// workgroups, as many as fit on the device at once (two per CU for both kernels), but
// keeps at least 4 chunks (256 entries) per workgroup: small prefixes are latency-bound,
// and spreading them wide pays for partials up to a quarter of the streamed bytes.  The
// kernel choice is made here once; the launch and the merge follow it.
Plan make_plan(int D, int Hq, const tv_state* st, int num_parts) {
  Plan p{};
  const int G = Hq / st->Hkv;
  p.R = G * D;
  p.mfma = st->dtype == TV_BF16 && st->d == 128;
  // the MFMA kernel takes more than 64 rows of a KV head (G*D > 64) in 128-row units of an
  // 8-wave workgroup, one per CU, so the rows share one stream of the prefix; the vector
  // kernel and smaller trees use 64-row units
  p.unit_rows = p.mfma && p.R > 64 ? 128 : 64;
  p.row_blocks = (p.R + p.unit_rows - 1) / p.unit_rows;
  p.tmax = 0;
  for (int l = 0; l < st->n_levels; ++l) p.tmax += (st->lvl[l].cap + 63) / 64;
  p.units = (long long)st->B * st->Hkv * p.row_blocks;
  const long long total = p.units * p.tmax;
  p.too_big = total > 0x7fffffffLL;
  if (total == 0 || p.too_big) {
    p.parts = 0;
  } else {
    long long want;
    const bool wide = p.unit_rows == 128;
    const long long slots = (long long)device_cus() * (wide ? 1 : 2);  // workgroups resident at once
    const long long pad = (long long)st->B * D;                        // scratch-pad workgroups
    // The scratch pad rides in the same launch (of 256-thread workgroups): ahead of the
    // stream's workgroups when the stream leaves room for it or when it is a handful of
    // workgroups (taken from the stream's), else behind them, where its short workgroups
    // fill the slots of the first slices to finish.
    if (num_parts > 0) {
      want = num_parts;
      p.fold = !wide && want + pad <= slots;
    } else {
      want = slots;
      const long long by_size = (total + 3) / 4;
      if (want > by_size) want = by_size;
      // A stream of 16 to 32 chunks per CU runs one slice per CU rather than two shorter
      // ones: each split slice writes a partial of one chunk's size that the merge reads back
      // (6% of a 16-chunk slice, 12% of an 8-chunk one).  Exactly one per CU: a few CUs with
      // two stream workgroups would finish last.  At batch 1 and a 131072-token prefix
      // (16.5 chunks per CU): 256 slices 40.3-40.6 us per call against 41.2-41.9 us for 504,
      // 43.9 us for 264.
      const long long cus = device_cus();
      if (!wide && total >= 16 * cus && total < 32 * cus && want > cus) want = cus;
      if (!wide && want + pad <= slots) {
        p.fold = true;
      } else if (!wide && pad <= 16 && pad < want) {
        want = slots - pad;
        p.fold = true;
      }
    }
    p.pad_after = !wide && !p.fold;
    if (want > total) want = total;
    if (want < 1) want = 1;
    // With at least one slice per unit, a multiple of the unit count puts every slice
    // boundary on a unit boundary or inside one unit, so no slice straddles two units
    // (each unit then has the same number of slices, and no workgroup starts a second
    // unit's prefix or writes two partials); taken when it keeps >= 7/8 of the slots.
    if (num_parts == 0 && want >= p.units) {
      const long long aligned = want / p.units * p.units;
      if (aligned * 8 >= want * 7) want = aligned;
    }
    p.parts = (int)want;  // slices of total / parts chunks, to within one (slice_begin)
    p.per_lo = total / want;
  }
  // Partials after long slices (8 chunks or more, i.e. long prefixes at small batch) are
  // written and read back with the nontemporal hint: measured 1-2 us faster per call at a
  // 131072-token prefix and batch 1, and 0.5-1 us slower after 4-chunk slices (batch 4-8 at
  // 4096-8192 tokens), whose partials the merge still finds in the caches.
  p.nt_partials = p.mfma && p.parts > 0 && p.per_lo >= 8;
  // the tail (< C0 tokens) and the D tree tokens form one extra chunk of at most 64
  // entries, attended in 16-entry tiles
  const int c0 = st->n_levels > 0 ? st->lvl[0].C : 1;
  const int tree_entries = D + (c0 - 1);
  p.fused_tree = p.mfma && p.parts > 0 && tree_entries <= 64;
  p.tree_tiles = tree_entries <= 16 ? 1 : tree_entries <= 32 ? 2 : 4;
  // every slice a whole number of units: each slice boundary a multiple of tmax (never with
  // more slices than units; always when the slice count divides the unit count; else checked
  // boundary by boundary)
  p.all_whole = p.fused_tree && p.parts > 0 && p.parts <= p.units;
  if (p.all_whole && p.units % p.parts != 0)
    for (long long q = 1; p.all_whole && q < p.parts; ++q) p.all_whole = q * total / p.parts % p.tmax == 0;
  // partials: one row block per (slice, unit) pair, numbered slice + unit
  const size_t rows = p.all_whole || p.parts == 0 ? 0 : (size_t)(p.parts + p.units - 1) * p.unit_rows;
  p.ws_o_bytes = round256(rows * st->d * sizeof(float));
  p.ws_ml_off = p.ws_o_bytes;
  p.total = p.ws_o_bytes + round256(rows * sizeof(float2));
  if (p.total == 0) p.total = 256;  // a workspace is always asked for (0 reports invalid arguments)
  return p;
}

// Branch-aware attention of D tree nodes (verify, or one draft-decode level); anc and
// depth rows are anc_ld long (the tree's first D nodes are the ones attended here).
tv_status run_attn(int D, int anc_ld, int Hq, const void* q, const void* k_tree, const void* v_tree,
                   const uint64_t* anc, const int32_t* depth, const int32_t* seq_err, const tv_state* st,
                   const tv_scratch* scratch, void* out, float* lse, void* workspace, size_t workspace_bytes,
                   int num_parts, hipStream_t stream) {
  tv_status s = check_state(st);
  if (s != TV_OK) return s;
  if (D < 1 || D > TV_MAX_D) return fail(TV_EINVAL, "D = %d outside 1..%d", D, TV_MAX_D);
  if (anc_ld < D || anc_ld > TV_MAX_D) return fail(TV_EINVAL, "anc_ld = %d outside D..%d", anc_ld, TV_MAX_D);
  if (Hq < 1 || Hq % st->Hkv != 0) return fail(TV_EINVAL, "Hq = %d is not a multiple of Hkv = %d", Hq, st->Hkv);
  if (num_parts < 0) return fail(TV_EINVAL, "num_parts = %d < 0", num_parts);
  if (st->B == 0) return ok();
  if (!q || !k_tree || !v_tree || !anc || !out) return fail(TV_EINVAL, "NULL pointer argument");
  if (scratch != nullptr && !depth) return fail(TV_EINVAL, "the scratch pad needs depth");
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out))
    return fail(TV_EINVAL, "q, k_tree, v_tree and out must be 16-byte aligned");
  if (scratch != nullptr) {
    tv_status sd = check_deferred(scratch, st);
    if (sd != TV_OK) return sd;
  }
  if (scratch != nullptr)
    for (int l = 0; l < st->n_levels; ++l) {
      if ((scratch->deferred >> l) & 1u) continue;  // no scratch states for this level
      if (!scratch->entry_k[l] || !scratch->entry_v[l] || !scratch->open_k[l] || !scratch->open_v[l])
        return fail(TV_EINVAL, "scratch level %d has a NULL pointer", l);
      if (!aligned16(scratch->entry_k[l]) || !aligned16(scratch->entry_v[l]) || !aligned16(scratch->open_k[l]) ||
          !aligned16(scratch->open_v[l]))
        return fail(TV_EINVAL, "scratch level %d must be 16-byte aligned", l);
    }
  const Plan p = make_plan(D, Hq, st, num_parts);
  if (p.too_big) return fail(TV_EUNSUPPORTED, "B * Hkv * row blocks * capacity chunks exceeds 2^31 - 1");
  if (workspace == nullptr || workspace_bytes < p.total)
    return fail(TV_EWORKSPACE, "workspace %zu bytes, need %zu", workspace == nullptr ? (size_t)0 : workspace_bytes,
                p.total);
  if (!aligned16(workspace)) return fail(TV_EINVAL, "workspace must be 16-byte aligned");

  tv::AttnArgs a{};
  a.B = st->B; a.D = D; a.Hq = Hq; a.Hkv = st->Hkv; a.d = st->d; a.G = Hq / st->Hkv; a.R = p.R;
  a.dtype = st->dtype; a.n_levels = st->n_levels;
  for (int l = 0; l < st->n_levels; ++l) {
    a.C[l] = st->lvl[l].C; a.cap[l] = st->lvl[l].cap;
    a.pk[l] = st->lvl[l].k; a.pvt[l] = st->lvl[l].vt; a.pn[l] = st->lvl[l].n;
    a.open_k[l] = st->lvl[l].open_k; a.open_v[l] = st->lvl[l].open_v;
    a.pt[l] = st->lvl[l].page_table; a.ppseq[l] = st->lvl[l].pages_per_seq; a.npages[l] = st->lvl[l].num_pages;
  }
  a.tail_k = st->tail_k; a.tail_v = st->tail_v; a.P = st->P;
  a.anc_ld = anc_ld;
  a.q = q; a.k_tree = k_tree; a.v_tree = v_tree; a.anc = anc; a.depth = depth; a.seq_err = seq_err;
  a.out = out; a.lse = lse;
  if (scratch != nullptr) a.scratch = *scratch;
  a.build_scratch = scratch != nullptr;
  a.unit_rows = p.unit_rows; a.row_blocks = p.row_blocks; a.tmax = p.tmax; a.units = (int)p.units; a.parts = p.parts;
  a.total = (int)(p.units * p.tmax);
  a.idx32 = (unsigned long long)p.parts * (unsigned long long)a.total < (1ull << 32);
  a.nt_partials = p.nt_partials;
  // slices touching one unit: its tmax chunks span at most (tmax - 1) / per_lo + 2 slices (a
  // bound of the slice length alone, so that batches cut the same way per unit merge alike)
  a.merge_nmax = p.parts > 0 ? (int)std::min<long long>(1 << 20, (p.tmax - 1) / p.per_lo + 2) : 0;
  a.ws_o = (float*)workspace;
  a.ws_ml = (float2*)((char*)workspace + p.ws_ml_off);
  a.scale_log2 = tv::kLog2e / std::sqrt((float)st->d);
  a.fused_tree = p.fused_tree;
  a.tree_tiles = p.tree_tiles;
  // the scratch pad needs only the tree tokens, the plan and the committed open sums: in
  // workgroups of the MFMA prefix launch when it has room, else a short kernel ahead of it
  a.fold_scratch = (p.mfma && (p.fold || p.pad_after) && p.parts > 0 && a.build_scratch && st->n_levels > 0)
                       ? st->B * D : 0;
  a.pad_after = a.fold_scratch > 0 && p.pad_after;
  if (a.fold_scratch == 0) {
    s = hip_check(tv::launch_scratch(a, stream), "scratch pad launch");
    if (s != TV_OK) return s;
  }
  s = hip_check(p.mfma ? tv::launch_attn_mfma(a, stream) : tv::launch_attn_valu(a, stream), "prefix attention launch");
  if (s != TV_OK) return s;
  // nothing left for the finish kernel when every slice is made of whole units: the
  // prefix kernel then wrote every output row itself
  if (p.all_whole) return ok();
  return hip_check(tv::launch_attn_finish(a, stream), "attention finish launch");
}

}  // namespace

extern "C" {

TV_API const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_EINVAL: return "invalid argument";
    case TV_EUNSUPPORTED: return "unsupported configuration";
    case TV_EWORKSPACE: return "workspace too small";
    case TV_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

TV_API const char* tv_last_error(void) { return g_err; }

TV_API int tv_version(void) { return TV_VERSION; }

TV_API tv_status tv_build_tree_mask(int B, int D, const int32_t* parents, uint64_t* anc, int32_t* depth,
                                    int32_t* seq_err, hipStream_t stream) {
  if (B < 0) return fail(TV_EINVAL, "B = %d < 0", B);
  if (D < 1 || D > TV_MAX_D) return fail(TV_EINVAL, "D = %d outside 1..%d", D, TV_MAX_D);
  if (B == 0) return ok();
  if (!parents || !anc || !depth || !seq_err) return fail(TV_EINVAL, "NULL pointer argument");
  return hip_check(tv::launch_tree_mask(B, D, parents, anc, depth, seq_err, stream), "tree mask launch");
}

TV_API tv_status tv_build_draft_tree(int B, int topk, int steps, int D, int vocab, const float* logits,
                                     const int32_t* root_tok, int32_t* parents, int32_t* draft_tok,
                                     float* cum_logp, hipStream_t stream) {
  if (B < 0) return fail(TV_EINVAL, "B = %d < 0", B);
  if (topk < 1 || steps < 1) return fail(TV_EINVAL, "topk = %d and steps = %d must be >= 1", topk, steps);
  if (vocab < topk) return fail(TV_EINVAL, "vocab = %d < topk = %d", vocab, topk);
  // E = 1 + k + ... + k^(steps-1) expanded nodes, N = k + ... + k^steps candidates
  long long E = 0, N = 0, width = 1;
  for (int l = 0; l < steps; ++l) {
    E += width;
    width *= topk;
    N += width;
    if (N > TV_DT_MAX_CAND)
      return fail(TV_EINVAL, "topk = %d, steps = %d create more than %d candidates", topk, steps, TV_DT_MAX_CAND);
  }
  const long long dmax = N + 1 < TV_MAX_D ? N + 1 : TV_MAX_D;
  if (D < 1 || D > dmax) return fail(TV_EINVAL, "D = %d outside 1..%lld", D, dmax);
  if ((long long)E * vocab > 0x7fffffffLL) return fail(TV_EINVAL, "E * vocab too large");
  if (B == 0) return ok();
  if (!logits || !root_tok || !parents || !draft_tok) return fail(TV_EINVAL, "NULL pointer argument");
  return hip_check(tv::launch_draft_tree(B, topk, steps, D, vocab, (int)E, (int)N, logits, root_tok, parents,
                                         draft_tok, cum_logp, stream),
                   "draft tree launch");
}

TV_API size_t tv_verify_attn_workspace_bytes(int D, int Hq, const tv_state* st, int num_parts) {
  if (D < 1 || D > TV_MAX_D || Hq < 1 || num_parts < 0) return 0;
  if (check_state(st) != TV_OK) return 0;
  if (Hq % st->Hkv != 0) return 0;
  const Plan p = make_plan(D, Hq, st, num_parts);
  return p.too_big ? 0 : p.total;
}

TV_API tv_status tv_verify_attn(int D, int Hq, const void* q, const void* k_tree, const void* v_tree,
                                const uint64_t* anc, const int32_t* depth, const int32_t* seq_err,
                                const tv_state* st, const tv_scratch* scratch, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, int num_parts,
                                hipStream_t stream) {
  if (depth == nullptr && st != nullptr && st->B > 0) return fail(TV_EINVAL, "NULL pointer argument (depth)");
  return run_attn(D, D, Hq, q, k_tree, v_tree, anc, depth, seq_err, st, scratch, out, lse, workspace,
                  workspace_bytes, num_parts, stream);
}

TV_API tv_status tv_verify_attn_noalloc(int D, int Hq, const void* q, const void* k_tree, const void* v_tree,
                                        const uint64_t* anc, const int32_t* depth, const int32_t* seq_err,
                                        const tv_state* st, const tv_scratch* scratch_pad, void* out, float* lse,
                                        int num_parts, hipStream_t stream) {
  if (depth == nullptr && st != nullptr && st->B > 0) return fail(TV_EINVAL, "NULL pointer argument (depth)");
  tv_status s = check_state(st);
  if (s != TV_OK) return s;
  if (D < 1 || D > TV_MAX_D) return fail(TV_EINVAL, "D = %d outside 1..%d", D, TV_MAX_D);
  if (Hq < 1 || Hq % st->Hkv != 0) return fail(TV_EINVAL, "Hq = %d is not a multiple of Hkv = %d", Hq, st->Hkv);
  if (num_parts < 0) return fail(TV_EINVAL, "num_parts = %d < 0", num_parts);
  const Plan plan = make_plan(D, Hq, st, num_parts);
  if (plan.too_big) return fail(TV_EUNSUPPORTED, "B * Hkv * row blocks * capacity chunks exceeds 2^31 - 1");
  const size_t need = plan.total;
  if (need > TV_NOALLOC_SCRATCH_BYTES)
    return fail(TV_EWORKSPACE, "this shape needs %zu bytes of split-prefix partials; tv_verify_attn_noalloc has %zu "
                "(use tv_verify_attn with a workspace, or more sequences per call so fewer prefixes are split)",
                need, (size_t)TV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  s = noalloc_scratch(&ws);
  if (s != TV_OK) return s;
  return run_attn(D, D, Hq, q, k_tree, v_tree, anc, depth, seq_err, st, scratch_pad, out, lse, ws,
                  TV_NOALLOC_SCRATCH_BYTES, num_parts, stream);
}

TV_API tv_status tv_draft_attn(int D, int anc_ld, int Hq, const void* q, const void* k_tree, const void* v_tree,
                               const uint64_t* anc, const int32_t* seq_err, const tv_state* st, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, int num_parts,
                               hipStream_t stream) {
  return run_attn(D, anc_ld, Hq, q, k_tree, v_tree, anc, nullptr, seq_err, st, nullptr, out, lse, workspace,
                  workspace_bytes, num_parts, stream);
}

TV_API tv_status tv_accept(int B, int D, const int32_t* parents, const uint64_t* anc, const int32_t* depth,
                           const int32_t* draft_tok, const int32_t* target_tok, const int32_t* seq_err,
                           int32_t* m, int32_t* path, int32_t* bonus, hipStream_t stream) {
  if (B < 0) return fail(TV_EINVAL, "B = %d < 0", B);
  if (D < 1 || D > TV_MAX_D) return fail(TV_EINVAL, "D = %d outside 1..%d", D, TV_MAX_D);
  if (B == 0) return ok();
  if (!parents || !anc || !depth || !draft_tok || !target_tok || !m || !path || !bonus)
    return fail(TV_EINVAL, "NULL pointer argument");
  return hip_check(tv::launch_accept(B, D, parents, anc, depth, draft_tok, target_tok, seq_err, m, path, bonus,
                                     stream),
                   "accept launch");
}

TV_API tv_status tv_refresh_state(int D, const tv_state* st, const tv_scratch* scratch, const void* k_tree,
                                  const void* v_tree, const int32_t* m, const int32_t* path,
                                  int32_t* commit_log, int32_t* seq_err, hipStream_t stream) {
  tv_status s = check_state(st);
  if (s != TV_OK) return s;
  if (D < 1 || D > TV_MAX_D) return fail(TV_EINVAL, "D = %d outside 1..%d", D, TV_MAX_D);
  if (st->B == 0) return ok();
  if (!k_tree || !v_tree || !m || !path || !seq_err) return fail(TV_EINVAL, "NULL pointer argument");
  tv_scratch sc{};
  if (st->n_levels > 0) {
    if (scratch == nullptr) return fail(TV_EINVAL, "scratch is NULL");
    s = check_deferred(scratch, st);
    if (s != TV_OK) return s;
    for (int l = 0; l < st->n_levels; ++l)
      if (!((scratch->deferred >> l) & 1u) &&
          (!scratch->entry_k[l] || !scratch->entry_v[l] || !scratch->open_k[l] || !scratch->open_v[l]))
        return fail(TV_EINVAL, "scratch level %d has a NULL pointer", l);
    sc = *scratch;
  }
  return hip_check(tv::launch_refresh(D, *st, sc, k_tree, v_tree, m, path, commit_log, seq_err, stream),
                   "refresh launch");
}

TV_API tv_status tv_accept_refresh(int D, const tv_state* st, const tv_scratch* scratch, const int32_t* parents,
                                   const uint64_t* anc, const int32_t* depth, const int32_t* draft_tok,
                                   const int32_t* target_tok, const void* k_tree, const void* v_tree, int32_t* m,
                                   int32_t* path, int32_t* bonus, int32_t* commit_log, int32_t* seq_err,
                                   hipStream_t stream) {
  tv_status s = check_state(st);
  if (s != TV_OK) return s;
  if (D < 1 || D > TV_MAX_D) return fail(TV_EINVAL, "D = %d outside 1..%d", D, TV_MAX_D);
  if (st->B == 0) return ok();
  if (!parents || !anc || !depth || !draft_tok || !target_tok || !k_tree || !v_tree || !m || !path || !bonus ||
      !seq_err)
    return fail(TV_EINVAL, "NULL pointer argument");
  tv_scratch sc{};
  if (st->n_levels > 0) {
    if (scratch == nullptr) return fail(TV_EINVAL, "scratch is NULL");
    s = check_deferred(scratch, st);
    if (s != TV_OK) return s;
    for (int l = 0; l < st->n_levels; ++l)
      if (!((scratch->deferred >> l) & 1u) &&
          (!scratch->entry_k[l] || !scratch->entry_v[l] || !scratch->open_k[l] || !scratch->open_v[l]))
        return fail(TV_EINVAL, "scratch level %d has a NULL pointer", l);
    sc = *scratch;
  }
  return hip_check(tv::launch_accept_refresh(D, *st, sc, parents, anc, depth, draft_tok, target_tok, k_tree, v_tree,
                                             m, path, bonus, commit_log, seq_err, stream),
                   "accept + refresh launch");
}

TV_API tv_status tv_compress_prefix(const tv_state* st, const void* raw_k, const void* raw_v, int max_len,
                                    int32_t* seq_err, hipStream_t stream) {
  tv_status s = check_state(st);
  if (s != TV_OK) return s;
  if (max_len < 0) return fail(TV_EINVAL, "max_len = %d < 0", max_len);
  if (st->B == 0) return ok();
  if (!seq_err) return fail(TV_EINVAL, "NULL seq_err");
  if (max_len > 0 && (!raw_k || !raw_v)) return fail(TV_EINVAL, "NULL raw prefix pointer");
  return hip_check(tv::launch_compress(*st, raw_k, raw_v, max_len, seq_err, stream), "compress launch");
}

}  // extern "C"
