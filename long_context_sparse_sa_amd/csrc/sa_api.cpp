// C ABI of the sparse-attention path: argument validation, workspace sizing and the launch sequences.
// Validation is pure host code and runs before any HIP call, so every error path is testable without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/sa.h"
#include "sa_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dt) { return dt == SA_F32 ? 4 : dt == SA_BF16 ? 2 : 1; }

bool valid_dtype(int dt) { return dt == SA_F32 || dt == SA_BF16 || dt == SA_E4M3; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Carves a workspace into 256-byte aligned pieces.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

int check_indexer(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld, int64_t L,
                  int32_t B, int32_t H, int32_t d) {
  if (!q || !w || !k) return fail(SA_ERR_NULL, "q, w and k must be non-NULL");
  if (!valid_dtype(q_dtype) || !valid_dtype(k_dtype)) return fail(SA_ERR_DTYPE, "unknown dtype");
  if (q_dtype != k_dtype) return fail(SA_ERR_DTYPE, "q and k must share one dtype (f32, bf16 or e4m3)");
  if (L < 1 || L > 0x7FFFFFFFLL) return fail(SA_ERR_SHAPE, "L must be in [1, 2^31)");
  if (B < 0 || H < 1 || d < 1) return fail(SA_ERR_SHAPE, "need B >= 0, H >= 1, d >= 1");
  if (k_ld < d) return fail(SA_ERR_SHAPE, "k_ld (%lld) < d (%d)", (long long)k_ld, d);
  if ((size_t)H * d > 16000) return fail(SA_ERR_SHAPE, "H * d must be <= 16000");
  if (!aligned16(q) || !aligned16(k) || !aligned16(w)) return fail(SA_ERR_ALIGN, "q, w and k must be 16-byte aligned");
  if ((k_ld * (int64_t)elem_size(k_dtype)) % 16 != 0) return fail(SA_ERR_ALIGN, "k rows must be 16-byte aligned");
  if (((int64_t)d * (int64_t)elem_size(q_dtype)) % 16 != 0) return fail(SA_ERR_ALIGN, "d * element size must be a multiple of 16");
  return SA_OK;
}

sa::IndexerArgs make_indexer(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                             int64_t L, int32_t B, int32_t H, int32_t d, const int32_t* t) {
  sa::IndexerArgs a;
  a.q = q;
  a.q_dtype = q_dtype;
  a.w = w;
  a.k = k;
  a.k_dtype = k_dtype;
  a.k_ld = k_ld;
  a.L = L;
  a.B = B;
  a.H = H;
  a.d = d;
  a.t = t;
  return a;
}

// ---- sa_select_topk plans -----------------------------------------------------------------------------------------
constexpr int64_t kFirstLevel = 16384;
constexpr int64_t kLevelGrowth = 8;
constexpr int kAutoPerQueryMinB = 64;

constexpr int64_t kAutoRadixMaxKeys = (int64_t)1 << 24;  // B * L up to which few queries take the radix select

int resolve_algo(int algo, const sa::IndexerArgs& a) {
  if (algo != SA_TOPK_AUTO) return algo;
  if (a.B >= kAutoPerQueryMinB && sa::stream_select_supported(a)) return SA_TOPK_PER_QUERY;
  // few queries: writing one key per position and selecting over all of them with every workgroup beats the
  // level-by-level thresholds until the key buffer gets large; beyond that the radix select takes a prefix and
  // its k-th key prunes the rest (measured faster than thresholds refined over geometric levels from 16K)
  return (int64_t)a.B * a.L <= kAutoRadixMaxKeys ? SA_TOPK_RADIX : SA_TOPK_RADIX_LEVELS;
}

struct RadixWs {
  sa::RadixPlan p;
  uint32_t* ctl;   // histograms, per-chunk counts and the chunk ticket (zeroed by the scoring launch)
  size_t ctl_words;
  uint32_t* keys;  // [B, keys_ld] one key per position
  size_t bytes;
};

RadixWs carve_radix(void* ws, const sa::IndexerArgs& a) {
  RadixWs w{};
  w.p = sa::radix_plan(a.B, a.L);
  Carver c(ws);
  w.ctl_words = sa::radix_ctl_words(a.B, w.p);
  w.ctl = c.take<uint32_t>(w.ctl_words);
  w.keys = c.take<uint32_t>((size_t)a.B * w.p.keys_ld);
  w.bytes = align_up(c.off, 256);
  return w;
}

// Level boundaries of the split-L algorithm: [0, first), [first, 8 first), ... up to L. The first level holds at least
// 4 k positions so that the first threshold already prunes.
// Key ranges after a radix-selected prefix [0, f): [f, 8 f), [8 f, 64 f), ... up to L (none when f >= L).
std::vector<int64_t> levels_after(int64_t f, int64_t L) {
  std::vector<int64_t> b{f};
  int64_t e = f * kLevelGrowth;
  while (e < L) {
    b.push_back(e);
    e *= kLevelGrowth;
  }
  if (f < L) b.push_back(L);
  return b;
}

std::vector<int64_t> levels(int64_t L, int k, int kpw) {
  int64_t first = kFirstLevel;
  if (first < 4 * (int64_t)k) first = 4 * (int64_t)k;
  first = (first + kpw - 1) / kpw * kpw;
  std::vector<int64_t> b{0};
  int64_t e = first;
  while (e < L) {
    b.push_back(e);
    e *= kLevelGrowth;
  }
  b.push_back(L);
  return b;
}

struct SplitLWs {
  uint32_t* thr;
  sa::Cand* kept;
  int32_t* kept_n;
  uint32_t* seg_cnt;     // [B, max_seg] per-workgroup candidate counts of the current key range
  sa::Cand* cand;        // [B, cand_ld] candidates of the current key range
  sa::Cand* gather;      // [B, gather_cap]
  int64_t cand_ld, gather_cap;
  int max_seg;
  size_t bytes;
};

// Workspace of a sequence of key ranges lv; first_slots: the first range writes one key per position (slots)
// instead of emitting into per-workgroup segments.
SplitLWs carve_levels(void* ws, const sa::IndexerArgs& a, int k, const std::vector<int64_t>& lv, bool first_slots) {
  int64_t max_level = 0;
  int max_seg = 1;
  for (size_t i = 0; i + 1 < lv.size(); ++i) {
    max_level = std::max(max_level, lv[i + 1] - lv[i]);
    if (i > 0 || !first_slots) max_seg = std::max(max_seg, sa::score_emit_plan(a, lv[i], lv[i + 1]).n_seg);
  }
  SplitLWs w{};
  w.cand_ld = (int64_t)align_up((size_t)max_level, 512);
  w.gather_cap = k + w.cand_ld;
  w.max_seg = max_seg;
  Carver c(ws);
  w.thr = c.take<uint32_t>(a.B);
  w.kept_n = c.take<int32_t>(a.B);
  w.seg_cnt = c.take<uint32_t>((size_t)a.B * max_seg);
  w.kept = c.take<sa::Cand>((size_t)a.B * k);
  w.cand = c.take<sa::Cand>((size_t)a.B * w.cand_ld);
  w.gather = c.take<sa::Cand>((size_t)a.B * w.gather_cap);
  w.bytes = align_up(c.off, 256);
  return w;
}

SplitLWs carve_split_l(void* ws, const sa::IndexerArgs& a, int k) {
  return carve_levels(ws, a, k, levels(a.L, k, sa::score_keys_per_wg(a)), true);
}

// The radix-selected prefix [0, f): at most half the positions and at most kAutoRadixMaxKeys keys over all
// queries, a multiple of the scoring workgroup's key count; a cache too short to split is selected whole.
int64_t radix_prefix(const sa::IndexerArgs& a) {
  const int64_t kpw = sa::score_keys_per_wg(a);
  int64_t f = std::min<int64_t>(kAutoRadixMaxKeys / std::max(a.B, 1), a.L / 2);
  f = f / kpw * kpw;
  return f >= kpw ? f : a.L;
}

struct RadixLevelsWs {
  int64_t prefix;
  std::vector<int64_t> lv;  // key ranges after the prefix
  RadixWs r;                // the prefix's radix select
  SplitLWs l;               // the ranges after it (kept list, threshold, candidates)
  size_t bytes;
};

RadixLevelsWs carve_radix_levels(void* ws, const sa::IndexerArgs& a, int k) {
  RadixLevelsWs w{};
  w.prefix = radix_prefix(a);
  sa::IndexerArgs ap = a;
  ap.L = w.prefix;
  w.r = carve_radix(ws, ap);
  w.lv = levels_after(w.prefix, a.L);
  w.l = carve_levels(ws ? static_cast<char*>(ws) + w.r.bytes : nullptr, a, k, w.lv, false);
  w.bytes = w.r.bytes + w.l.bytes;
  return w;
}

struct PerQueryWs {
  sa::Cand* buf;
  int32_t* buf_n;
  sa::Cand* gather;
  int cap;
  size_t bytes;
};

PerQueryWs carve_per_query(void* ws, const sa::IndexerArgs& a, int k) {
  PerQueryWs w{};
  w.cap = (int)align_up((size_t)4 * k + 64, 64);  // a larger buffer means fewer compactions per query
  Carver c(ws);
  w.buf_n = c.take<int32_t>(a.B);
  w.buf = c.take<sa::Cand>((size_t)a.B * w.cap);
  w.gather = c.take<sa::Cand>((size_t)a.B * w.cap);
  w.bytes = align_up(c.off, 256);
  return w;
}

}  // namespace

extern "C" {

SA_API const char* sa_status_string(int s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL: return "SA_ERR_NULL";
    case SA_ERR_SHAPE: return "SA_ERR_SHAPE";
    case SA_ERR_DTYPE: return "SA_ERR_DTYPE";
    case SA_ERR_ALIGN: return "SA_ERR_ALIGN";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    default: return "SA_ERR_UNKNOWN";
  }
}

SA_API const char* sa_last_error(void) { return g_err; }

SA_API int sa_version(void) { return 1; }

// ---------------------------------------------------------------------------------------------------------------
SA_API int sa_index_score(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d, const int32_t* t, int64_t s_begin,
                          int64_t s_end, float* scores, int64_t scores_ld, void* stream) {
  int st = check_indexer(q, q_dtype, w, k, k_dtype, k_ld, L, B, H, d);
  if (st) return st;
  if (!scores) return fail(SA_ERR_NULL, "scores must be non-NULL");
  if (s_begin < 0 || s_end < s_begin || s_end > L) return fail(SA_ERR_SHAPE, "need 0 <= s_begin <= s_end <= L");
  if (scores_ld < s_end - s_begin) return fail(SA_ERR_SHAPE, "scores_ld < s_end - s_begin");
  if (B == 0 || s_end == s_begin) return SA_OK;
  const sa::IndexerArgs a = make_indexer(q, q_dtype, w, k, k_dtype, k_ld, L, B, H, d, t);
  hipError_t e = sa::launch_score(a, s_begin, s_end, sa::kScoreDense, scores, scores_ld, 0, 0, nullptr, nullptr, 0,
                                  nullptr, (hipStream_t)stream);
  return e == hipSuccess ? SA_OK : hip_fail(e, "sa_index_score");
}

// ---------------------------------------------------------------------------------------------------------------
SA_API size_t sa_select_topk_workspace(int64_t L, int32_t B, int32_t H, int32_t d, int q_dtype, int k_dtype,
                                       int32_t k_sparse, int algo) {
  if (L < 1 || B < 0 || H < 1 || d < 1 || k_sparse < 1) return 0;
  const sa::IndexerArgs a = make_indexer(nullptr, q_dtype, nullptr, nullptr, k_dtype, d, L, B, H, d, nullptr);
  const int alg = resolve_algo(algo, a);
  if (alg == SA_TOPK_PER_QUERY) return carve_per_query(nullptr, a, k_sparse).bytes;
  if (alg == SA_TOPK_RADIX) return carve_radix(nullptr, a).bytes;
  if (alg == SA_TOPK_RADIX_LEVELS) return carve_radix_levels(nullptr, a, k_sparse).bytes;
  return carve_split_l(nullptr, a, k_sparse).bytes;
}

SA_API int sa_select_topk(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d, const int32_t* t, int32_t k_sparse,
                          int32_t n_sink, int32_t n_window, int32_t* idx, int32_t idx_ld, int32_t* n_sel, void* ws,
                          size_t ws_bytes, int algo, void* stream) {
  int st = check_indexer(q, q_dtype, w, k, k_dtype, k_ld, L, B, H, d);
  if (st) return st;
  if (!idx || !n_sel) return fail(SA_ERR_NULL, "idx and n_sel must be non-NULL");
  if (k_sparse < 1 || k_sparse > sa::merge_max_k())
    return fail(SA_ERR_SHAPE, "k_sparse must be in [1, %d]", sa::merge_max_k());
  if (idx_ld < k_sparse) return fail(SA_ERR_SHAPE, "idx_ld (%d) < k_sparse (%d)", idx_ld, k_sparse);
  if (n_sink < 0 || n_window < 0) return fail(SA_ERR_SHAPE, "n_sink and n_window must be >= 0");
  if (algo < SA_TOPK_AUTO || algo > SA_TOPK_RADIX_LEVELS) return fail(SA_ERR_SHAPE, "unknown algo %d", algo);
  const sa::IndexerArgs a = make_indexer(q, q_dtype, w, k, k_dtype, k_ld, L, B, H, d, t);
  const int alg = resolve_algo(algo, a);
  if (alg == SA_TOPK_PER_QUERY && !sa::stream_select_supported(a))
    return fail(SA_ERR_UNSUPPORTED, "the per-query algorithm needs d = 128, H in {32, 64} and bf16 or e4m3 inputs");
  const size_t need = sa_select_topk_workspace(L, B, H, d, q_dtype, k_dtype, k_sparse, alg);
  if (!ws || ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (!aligned16(ws)) return fail(SA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (B == 0) return SA_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (alg == SA_TOPK_PER_QUERY) {
    const PerQueryWs w2 = carve_per_query(ws, a, k_sparse);
    e = sa::launch_stream_select(a, k_sparse, n_sink, n_window, w2.buf, w2.buf_n, w2.cap, s);
    if (e != hipSuccess) return hip_fail(e, "sa_select_topk (stream)");
    sa::MergeIn in{};
    in.kept = w2.buf;
    in.kept_ld = w2.cap;
    in.kept_n = w2.buf_n;
    sa::MergeOut out{};
    out.final_mode = 1;
    out.idx = idx;
    out.idx_ld = idx_ld;
    out.n_sel = n_sel;
    e = sa::launch_merge(B, k_sparse, in, w2.gather, w2.cap, out, s);
    return e == hipSuccess ? SA_OK : hip_fail(e, "sa_select_topk (final merge)");
  }
  if (alg == SA_TOPK_RADIX) {
    // every position's key into the workspace (0 for positions outside the candidate range), then the radix
    // select over all of them
    const RadixWs w2 = carve_radix(ws, a);
    sa::IndexerArgs as = a;
    as.clear = w2.ctl;  // the scoring launch zeroes the select's counters
    as.clear_n = (int64_t)w2.ctl_words;
    e = sa::launch_score(as, 0, L, sa::kScoreAll, nullptr, 0, n_sink, n_window, nullptr,
                         reinterpret_cast<sa::Cand*>(w2.keys), w2.p.keys_ld, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "sa_select_topk (radix score)");
    e = sa::launch_radix_select(B, L, k_sparse, w2.p, w2.keys, w2.ctl, idx, idx_ld, n_sel, nullptr, nullptr, s);
    return e == hipSuccess ? SA_OK : hip_fail(e, "sa_select_topk (radix select)");
  }
  if (alg == SA_TOPK_RADIX_LEVELS) {
    // the exact top-k of the prefix by the radix select, kept as (key, position) pairs with its k-th key as the
    // threshold; then each later key range emits only keys above the threshold and a merge keeps the k best
    const RadixLevelsWs w2 = carve_radix_levels(ws, a, k_sparse);
    const bool whole = w2.prefix >= L;
    sa::IndexerArgs as = a;
    as.clear = w2.r.ctl;  // the scoring launch zeroes the select's counters
    as.clear_n = (int64_t)w2.r.ctl_words;
    e = sa::launch_score(as, 0, w2.prefix, sa::kScoreAll, nullptr, 0, n_sink, n_window, nullptr,
                         reinterpret_cast<sa::Cand*>(w2.r.keys), w2.r.p.keys_ld, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "sa_select_topk (prefix score)");
    e = sa::launch_radix_select(B, w2.prefix, k_sparse, w2.r.p, w2.r.keys, w2.r.ctl, whole ? idx : nullptr, idx_ld,
                                whole ? n_sel : w2.l.kept_n, whole ? nullptr : w2.l.kept,
                                whole ? nullptr : w2.l.thr, s);
    if (e != hipSuccess) return hip_fail(e, "sa_select_topk (prefix select)");
    for (size_t i = 0; i + 1 < w2.lv.size(); ++i) {
      const int64_t lo = w2.lv[i], hi = w2.lv[i + 1];
      e = sa::launch_score(a, lo, hi, sa::kScoreEmit, nullptr, 0, n_sink, n_window, w2.l.thr, w2.l.cand,
                           w2.l.cand_ld, w2.l.seg_cnt, s);
      if (e != hipSuccess) return hip_fail(e, "sa_select_topk (score)");
      sa::MergeIn in{};
      in.kept = w2.l.kept;
      in.kept_ld = k_sparse;
      in.kept_n = w2.l.kept_n;
      in.cand = w2.l.cand;
      in.cand_ld = w2.l.cand_ld;
      const sa::EmitPlan ep = sa::score_emit_plan(a, lo, hi);
      in.seg_cnt = w2.l.seg_cnt;
      in.n_seg = ep.n_seg;
      in.seg_cap = ep.seg_cap;
      sa::MergeOut out{};
      out.final_mode = i + 2 == w2.lv.size() ? 1 : 0;
      out.kept_out = w2.l.kept;
      out.kept_n_out = w2.l.kept_n;
      out.thr_out = w2.l.thr;
      out.idx = idx;
      out.idx_ld = idx_ld;
      out.n_sel = n_sel;
      e = sa::launch_merge(B, k_sparse, in, w2.l.gather, w2.l.gather_cap, out, s);
      if (e != hipSuccess) return hip_fail(e, "sa_select_topk (merge)");
    }
    return SA_OK;
  }
  const SplitLWs w2 = carve_split_l(ws, a, k_sparse);
  const int kpw = sa::score_keys_per_wg(a);
  const std::vector<int64_t> lv = levels(L, k_sparse, kpw);
  // Key ranges in ascending position order. The first range writes every candidate to its position's slot; later
  // ranges write only candidates above the k-th key kept so far, each workgroup into its own segment. Every merge
  // keeps its input order, so the kept lists and the final index lists stay in ascending position order.
  for (size_t i = 0; i + 1 < lv.size(); ++i) {
    const int64_t lo = lv[i], hi = lv[i + 1];
    const bool first = i == 0, last = i + 2 == lv.size();
    e = sa::launch_score(a, lo, hi, first ? sa::kScoreAll : sa::kScoreEmit, nullptr, 0, n_sink, n_window,
                         first ? nullptr : w2.thr, w2.cand, w2.cand_ld, first ? nullptr : w2.seg_cnt, s);
    if (e != hipSuccess) return hip_fail(e, "sa_select_topk (score)");
    sa::MergeIn in{};
    in.kept = first ? nullptr : w2.kept;
    in.kept_ld = k_sparse;
    in.kept_n = w2.kept_n;
    if (first) {
      in.slot_key = reinterpret_cast<const uint32_t*>(w2.cand);
      in.slot_ld = w2.cand_ld;
      in.n_slots = hi - lo;
      in.slot_pos0 = (int32_t)lo;
    } else {
      in.cand = w2.cand;
      in.cand_ld = w2.cand_ld;
      const sa::EmitPlan ep = sa::score_emit_plan(a, lo, hi);
      in.seg_cnt = w2.seg_cnt;
      in.n_seg = ep.n_seg;
      in.seg_cap = ep.seg_cap;
    }
    sa::MergeOut out{};
    out.final_mode = last ? 1 : 0;
    out.kept_out = w2.kept;
    out.kept_n_out = w2.kept_n;
    out.thr_out = w2.thr;
    out.idx = idx;
    out.idx_ld = idx_ld;
    out.n_sel = n_sel;
    e = sa::launch_merge(B, k_sparse, in, w2.gather, w2.gather_cap, out, s);
    if (e != hipSuccess) return hip_fail(e, "sa_select_topk (merge)");
  }
  return SA_OK;
}

// ---------------------------------------------------------------------------------------------------------------
SA_API size_t sa_bucket_build_workspace(int64_t L, int32_t n_buckets) {
  if (L < 0 || n_buckets < 1) return 0;
  const sa::BucketBuildPlan p = sa::bucket_build_plan(L, n_buckets);
  Carver c(nullptr);
  c.take<int32_t>(n_buckets);
  c.take<int32_t>((size_t)p.n_chunks * n_buckets);
  return align_up(c.off, 256);
}

SA_API int sa_bucket_build(const void* k, int k_dtype, int64_t k_ld, int64_t L, int32_t d, const int32_t* assign,
                           int32_t n_buckets, float* reps, int32_t* offsets, int32_t* members, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!k || !assign || !reps || !offsets || !members) return fail(SA_ERR_NULL, "k, assign, reps, offsets, members must be non-NULL");
  if (k_dtype != SA_F32 && k_dtype != SA_BF16) return fail(SA_ERR_DTYPE, "bucket keys must be f32 or bf16");
  if (L < 1 || L > 0x7FFFFFFFLL || d < 1 || n_buckets < 1) return fail(SA_ERR_SHAPE, "need 1 <= L < 2^31, d >= 1, n_buckets >= 1");
  if (k_ld < d) return fail(SA_ERR_SHAPE, "k_ld < d");
  const size_t need = sa_bucket_build_workspace(L, n_buckets);
  if (!ws || ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  const sa::BucketBuildPlan p = sa::bucket_build_plan(L, n_buckets);
  Carver c(ws);
  int32_t* counts = c.take<int32_t>(n_buckets);
  int32_t* table = c.take<int32_t>((size_t)p.n_chunks * n_buckets);
  hipError_t e = sa::launch_bucket_build(k, k_dtype, k_ld, L, d, assign, n_buckets, reps, offsets, members, counts,
                                         table, p, (hipStream_t)stream);
  return e == hipSuccess ? SA_OK : hip_fail(e, "sa_bucket_build");
}

SA_API size_t sa_bucket_select_workspace(int32_t B, int32_t n_buckets, int32_t top_b) {
  if (B < 0 || n_buckets < 1 || top_b < 1) return 0;
  Carver c(nullptr);
  c.take<uint32_t>((size_t)B * n_buckets);  // one score key per (query, bucket)
  return align_up(c.off, 256);
}

SA_API int sa_bucket_select(const void* q, int q_dtype, int32_t B, int32_t d, const float* reps,
                            const int32_t* offsets, const int32_t* members, int32_t n_buckets, int64_t L,
                            const int32_t* t, int32_t top_b, int32_t n_sink, int32_t n_window, int32_t* idx,
                            int32_t cap, int32_t* n_sel, int32_t* buckets_out, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!q || !reps || !offsets || !members || !idx || !n_sel) return fail(SA_ERR_NULL, "required pointer is NULL");
  if (q_dtype != SA_F32 && q_dtype != SA_BF16) return fail(SA_ERR_DTYPE, "bucket queries must be f32 or bf16");
  if (B < 0 || d < 1 || n_buckets < 1 || L < 1 || L > 0x7FFFFFFFLL) return fail(SA_ERR_SHAPE, "bad B, d, n_buckets or L");
  if ((size_t)B * d > 16000) return fail(SA_ERR_SHAPE, "B * d must be <= 16000");
  if (top_b < 1 || top_b > n_buckets || top_b > 1024) return fail(SA_ERR_SHAPE, "need 1 <= top_b <= min(n_buckets, 1024)");
  if (cap < 1 || cap > sa::bucket_expand_max()) return fail(SA_ERR_SHAPE, "cap must be in [1, %d]", sa::bucket_expand_max());
  if (n_sink < 0 || n_window < 0) return fail(SA_ERR_SHAPE, "n_sink and n_window must be >= 0");
  const size_t need = sa_bucket_select_workspace(B, n_buckets, top_b);
  if (!ws || ws_bytes < need) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (B == 0) return SA_OK;
  Carver c(ws);
  uint32_t* keys = c.take<uint32_t>((size_t)B * n_buckets);
  hipError_t e = sa::launch_bucket_select(q, q_dtype, B, d, reps, offsets, members, n_buckets, L, t, top_b, n_sink,
                                          n_window, idx, cap, n_sel, buckets_out, keys, (hipStream_t)stream);
  return e == hipSuccess ? SA_OK : hip_fail(e, "sa_bucket_select");
}

// ---------------------------------------------------------------------------------------------------------------
SA_API size_t sa_sparse_attn_workspace(int32_t B, int32_t H, int32_t d_qk, int32_t d_v, int64_t max_rows, int dtype) {
  if (B < 0 || H < 1 || d_qk < 1 || d_v < 1 || max_rows < 0) return 0;
  return align_up(sa::attn_workspace_bound(B, H, d_qk, d_v, max_rows, dtype), 256);
}

SA_API int sa_sparse_attn(const void* q, const void* kv, const void* v, int dtype, int64_t kv_ld, int64_t v_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d_qk, int32_t d_v, const int32_t* t,
                          const int32_t* idx, int32_t idx_ld, const int32_t* n_sel, int32_t n_sink,
                          int32_t n_window, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!q || !kv || !out) return fail(SA_ERR_NULL, "q, kv and out must be non-NULL");
  if ((idx == nullptr) != (n_sel == nullptr)) return fail(SA_ERR_NULL, "idx and n_sel must be both NULL or both set");
  if (dtype != SA_F32 && dtype != SA_BF16) return fail(SA_ERR_DTYPE, "attention dtype must be f32 or bf16");
  if (L < 1 || L > 0x7FFFFFFFLL || B < 0 || H < 1 || d_qk < 1 || d_v < 1)
    return fail(SA_ERR_SHAPE, "need 1 <= L < 2^31, B >= 0, H, d_qk, d_v >= 1");
  if (kv_ld < d_qk || (!v && kv_ld < d_v) || (v && v_ld < d_v)) return fail(SA_ERR_SHAPE, "leading dimension too small");
  if (d_v > 1024 || d_qk > 16000) return fail(SA_ERR_SHAPE, "need d_v <= 1024 and d_qk <= 16000");
  if (idx_ld < 0 || n_sink < 0 || n_window < 0) return fail(SA_ERR_SHAPE, "idx_ld, n_sink, n_window must be >= 0");
  if (!std::isfinite(scale)) return fail(SA_ERR_SHAPE, "scale must be finite");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || (v && !aligned16(v)))
    return fail(SA_ERR_ALIGN, "q, kv, v and out must be 16-byte aligned");
  const int64_t max_rows = (int64_t)n_sink + n_window + (idx ? idx_ld : 0);
  sa::AttnPlan p = sa::attn_plan(B, H, d_qk, d_v, max_rows, dtype, v != nullptr);
  if (p.mfma && (kv_ld % 8) != 0) p = sa::attn_plan(B, H, d_qk, d_v, max_rows, dtype, true);
  const size_t need = sa::attn_workspace_bytes(p, B, H, d_v);
  if (need > 0 && (!ws || ws_bytes < need)) return fail(SA_ERR_WORKSPACE, "workspace needs %zu bytes", need);
  if (B == 0) return SA_OK;
  sa::AttnArgs a;
  a.q = q;
  a.kv = kv;
  a.v = v;
  a.dtype = dtype;
  a.kv_ld = kv_ld;
  a.v_ld = v_ld;
  a.L = L;
  a.B = B;
  a.H = H;
  a.d_qk = d_qk;
  a.d_v = d_v;
  a.t = t;
  a.idx = idx;
  a.idx_ld = idx_ld;
  a.n_sel = n_sel;
  a.n_sink = n_sink;
  a.n_window = n_window;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  hipError_t e = sa::launch_attn(a, p, ws, (hipStream_t)stream);
  return e == hipSuccess ? SA_OK : hip_fail(e, "sa_sparse_attn");
}

}  // extern "C"
