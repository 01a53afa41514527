// Internal launch interface between the C ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

// Instrumentation: records the next event of the caller's stage-event list (sa_set_stage_events) on `st`, if a list
// is set on this thread and not used up. Every kernel launch of the library is followed by one call.
void stage_mark(hipStream_t st);

#define SA_NTH_5(a, b, c, d, e, ...) e
// A kernel launch followed by its stage mark (the fifth argument of hipLaunchKernelGGL is the stream).
#define SA_LAUNCH(...)                                \
  do {                                               \
    hipLaunchKernelGGL(__VA_ARGS__);                 \
    ::sa::stage_mark(SA_NTH_5(__VA_ARGS__, 0, 0, 0, 0, 0)); \
  } while (0)

struct IndexerArgs {
  const void* q;     // [B, H, d]
  int q_dtype;
  const float* w;    // [B, H]
  const void* k;     // [L, k_ld]
  int k_dtype;
  int64_t k_ld;
  int64_t L;
  int B, H, d;
  const int32_t* t;  // [B] or NULL
  // Optional: the scoring launch also zeroes clear[0, clear_n) (counters a following kernel accumulates into;
  // saves a separate fill launch).
  uint32_t* clear = nullptr;
  int64_t clear_n = 0;
  // Block maxima only: the B rows are (query, group) pairs, two 32-head groups per 64-head query, which one wave
  // scores together (the query's t is row 2 b's).
  bool groups2 = false;
};

// One emitted candidate: (order-preserving key of the fp32 score, position).
struct Cand {
  uint32_t key;
  int32_t pos;
};

enum ScoreMode { kScoreDense = 0, kScoreEmit = 1, kScoreAll = 2, kScorePage = 3, kScoreBlockMax = 4 };

// Positions handled by one workgroup of the scoring kernel chosen for these arguments.
int score_keys_per_wg(const IndexerArgs& a);
// True when the MFMA scoring kernel serves these arguments.
bool score_uses_mfma(const IndexerArgs& a);

// Segmented emission: workgroup w of a kScoreEmit launch scores a contiguous run of positions and appends its
// candidates, in ascending position order, to its own segment cand[b * cand_ld + w * seg_cap + ...]; it then
// stores the count in seg_cnt[b * n_seg + w]. No atomics, so the concatenated segments are in ascending order.
struct EmitPlan {
  int n_seg;        // workgroups per query = segments per query
  int64_t seg_cap;  // positions per workgroup = segment capacity
};
EmitPlan score_emit_plan(const IndexerArgs& a, int64_t lo, int64_t hi);

// Scores positions [lo, hi).
//  kScoreDense: scores[b * scores_ld + (s - lo)] = I(b, s), or -inf for s > t_b.
//  kScoreAll:   the cand buffer is read as uint32 keys: keys[b * cand_ld + (s - lo)] = score_key(I) for candidates s
//               (n_sink <= s <= t_b - n_window), 0 otherwise (the position is the slot's index).
//  kScoreEmit:  candidates with score_key(I) > thr_key[b] (any candidate when thr_key is NULL) go to the segments
//               described by score_emit_plan(a, lo, hi); seg_cnt receives the per-segment counts.
hipError_t launch_score(const IndexerArgs& a, int64_t lo, int64_t hi, int mode, float* scores, int64_t scores_ld,
                        int n_sink, int n_window, const uint32_t* thr_key, Cand* cand, int64_t cand_ld,
                        uint32_t* seg_cnt, hipStream_t stream);

// Candidates of one exact top-k merge, per query b, in this order:
//   kept:     kept[b * kept_ld + (0:kept_n[b])]                                   (when kept != NULL)
//   slots:    keys slot_key[b * slot_ld + i], i < n_slots, for position slot_pos0 + i; key 0 marks an empty
//             slot                                                              (when slot_key != NULL)
//   segments: seg_cnt[b * n_seg + w] entries at cand[b * cand_ld + w * seg_cap], w = 0, 1, ...  (when seg_cnt)
// The merge preserves this order. When the entries come in ascending position order, as every producer in this
// library writes them, the selected positions come out ascending without a sort.
struct MergeIn {
  const Cand* kept;
  int kept_ld;
  const int32_t* kept_n;
  const uint32_t* slot_key;
  int64_t slot_ld;
  int64_t n_slots;
  int32_t slot_pos0;
  const Cand* cand;
  int64_t cand_ld;
  const uint32_t* seg_cnt;
  int n_seg;
  int64_t seg_cap;
};
// final_mode 0: kept_out[b * k + (0:take)] = the k best (key desc, pos asc) in input order, kept_n_out[b] = take,
//               thr_out[b] = the k-th key (0 when there are fewer than k candidates);
// final_mode 1: idx[b, 0:take) = their positions in input order, -1 up to idx_ld, n_sel[b] = take;
// final_mode 2: idx[b, 0:take) = their positions in (key desc, position asc) order (bucket ranking).
struct MergeOut {
  int final_mode;
  Cand* kept_out;
  int32_t* kept_n_out;
  uint32_t* thr_out;
  int32_t* idx;
  int idx_ld;
  int32_t* n_sel;
};
// `gather` must hold, per query, every candidate of the merge (kept plus slots or segment entries): it stores
// them when they do not fit in LDS.
hipError_t launch_merge(int B, int k, const MergeIn& in, Cand* gather, int64_t gather_cap, const MergeOut& out,
                        hipStream_t stream);
int merge_max_k();
// Fills p[0, n) with v (a kernel, so that it is safe inside captured graphs).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);

// Radix select over all positions for few queries (k_radix.hip). keys[b * keys_ld + s] (s < L) hold the
// all-slots keys of the scoring kernel; the rest of each row is never read past the next multiple of 4.
// ctl holds radix_ctl_words(B, plan) words and must be zero on entry (the pass histograms, the per-chunk counts
// and the chunk ticket).
struct RadixPlan {
  int64_t keys_ld;  // row stride of keys (a multiple of 1024)
  int64_t chunk;    // positions per workgroup
  int n_chunks;     // workgroups per query
};
RadixPlan radix_plan(int B, int64_t L);
size_t radix_ctl_words(int B, const RadixPlan& p);
// The selection goes to idx (positions, -1 padded to idx_ld) and/or kept ([B, k] (key, position) pairs), either
// may be NULL; n_sel[b] = min(k, candidates); thr_out (or NULL) receives the k-th key (0 with fewer candidates).
hipError_t launch_radix_select(int B, int64_t L, int k, const RadixPlan& p, const uint32_t* keys, uint32_t* ctl,
                               int32_t* idx, int idx_ld, int32_t* n_sel, Cand* kept, uint32_t* thr_out,
                               hipStream_t stream);
// The radix select's keys from caller-given fp32 scores: keys[b * p.keys_ld + s] = score_key(scores[b, s]) for
// candidates (n_sink <= s <= t_b - n_window), 0 otherwise; also zeroes ctl[0, ctl_words).
// With t_div > 1 (page selection), entry s is a candidate when s <= (t_b / t_div) - n_window, t_b from t or
// t_default.
hipError_t launch_keys_from_scores(const float* scores, int64_t scores_ld, int64_t L, int B, const int32_t* t,
                                   int n_sink, int n_window, const RadixPlan& p, uint32_t* keys, uint32_t* ctl,
                                   int64_t ctl_words, hipStream_t stream, int64_t t_default = -1, int t_div = 1);

// Streaming selection for few queries (decode): launches over co-resident ranges of positions; each keeps its keys
// on chip, publishes per-chunk statistics, derives a lower bound T of each query's k-th key from them and emits only
// keys >= T into per-workgroup segments (one segment per workgroup and launch) for a final merge.
struct StreamPlan {
  int64_t end;       // positions [0, end) are scored
  int nq;            // queries per workgroup
  int run_keys;      // positions per workgroup (a multiple of 64) = segment capacity
  int64_t slots;     // workgroups (= statistics slots = segments) per query over all launches
  int64_t pub_ld;    // words per query row of the statistics area: one slot per workgroup of the call
  int top_words;     // words per query of the kept-statistics sketch
};
bool stream_supported(const IndexerArgs& a);
StreamPlan stream_plan(const IndexerArgs& a, int64_t end);
// pub [B, p.pub_ld] 32-bit slots (zeroed before the call's first launch); thr [B]; top [B, p.top_words];
// seg_cnt [B, p.slots]; cand [B, p.slots * p.run_keys]. spin_limit: polls of the other workgroups' publication
// before going on without them.
hipError_t launch_stream_decode(const IndexerArgs& a, int k, int n_sink, int n_window, const StreamPlan& p,
                                uint32_t* pub, uint32_t* thr, uint32_t* top, uint32_t* seg_cnt, Cand* cand,
                                int spin_limit, hipStream_t stream);

// ---- hierarchical index ------------------------------------------------------------------------------------------
// Sub-block mean keys: means[n, 0:d] = bf16(float(fp64 sum of k[n B + i, 0:d] over the block's cached positions /
// their count)) for n < ceil(L / B); keys bf16.
hipError_t launch_hi_means(const uint16_t* k, int64_t k_ld, int64_t L, int d, int sub, uint16_t* means,
                           hipStream_t stream);
// Page scores over the mean keys m (m.k = means, m.L = their count, m.t = the queries' token t): scores[b, p] = sum
// of the indexer score of the page_subs mean keys of page p (page_subs a power of two <= 64), -inf when the page's
// first position p * page_len is past t_b (t_b = tok_L - 1 without t).
hipError_t launch_page_scores(const IndexerArgs& m, int page_subs, int page_len, int64_t tok_L, float* scores,
                              int64_t scores_ld, hipStream_t stream);
// Token stage: per query, its recalled pages pages[b, 0:n_pages[b]) (ascending). The cache's pages are cut into
// n_parts ranges of part_pages page ids; one wave per (query, part) keeps, in segment seg[(b n_parts + part)
// seg_cap ...] with seg_cnt[b n_parts + part] entries, at most k candidates (in its pages, inside the sink/window
// budget, ascending positions) that contain the part's exact top-k: the merge's segment input.
constexpr int kHiMaxPages = 1 << 20;            // recalled pages per query (the size of the page list only)
constexpr int64_t kHiTargetWaves = 1536;        // (query, part) waves wanted at the least
struct HiFinePlan {
  int n_parts;
  int part_pages;
  int64_t seg_cap;
};
HiFinePlan hi_fine_plan(int64_t L, int B, int page_len, int k);
bool hi_fine_supported(const IndexerArgs& a);
hipError_t launch_hi_fine(const IndexerArgs& a, const int32_t* pages, int pages_ld, const int32_t* n_pages,
                          int page_len, int k, int n_sink, int n_window, const HiFinePlan& p, Cand* seg,
                          uint32_t* seg_cnt, hipStream_t stream);

// Block-granular indexers (k_blocks.hip and the MFMA scorer's block-max mode).
// keys[b * keys_ld + n] = max over positions s of block n (positions [n c, (n + 1) c)) of score_key(I(b, s)), for
// the blocks before the one holding t_b; the other entries are left as they are (zero them first). c is a
// multiple of 64. The MFMA scorer shapes only.
hipError_t launch_block_max(const IndexerArgs& a, int block, uint32_t* keys, int64_t keys_ld, hipStream_t stream);
// t_out[b * reps + r] = t ? t[b] : L - 1 (r < reps), then, with div > 1, max(0, (t + 1) / div - 1): the last complete
// micro-block of query b (clamped to 0 when there is none).
hipError_t launch_block_t(const int32_t* t, int B, int reps, int64_t L, int div, int32_t* t_out, hipStream_t stream);
// Micro-blocks of b positions to positions: the chosen blocks blk[q, 0:min(n_blk[q], kb)) (ascending), expanded,
// then the unfinished block's visible positions; no block when query q has no complete block.
hipError_t launch_qsa_expand(const int32_t* blk, int kb, const int32_t* n_blk, const int32_t* t, int B, int64_t L,
                             int b, int32_t* idx, int idx_ld, int32_t* n_sel, hipStream_t stream);
// Blocks of c positions to positions: the chosen earlier blocks blk[q, 0:n_blk[q]) (ascending; n_blk NULL: none)
// expanded, then the local block up to t[q].
hipError_t launch_msa_expand(const int32_t* blk, int blk_ld, const int32_t* n_blk, const int32_t* t, int B, int c,
                             int32_t* idx, int idx_ld, int32_t* n_sel, hipStream_t stream);

// Streaming per-query selection for many queries (prefill chunk): one pass over each query's visible keys keeps
// at most `cap` candidates per query in buf[b, :] (count in buf_n[b]) that contain the exact top-k.
bool stream_select_supported(const IndexerArgs& a);
hipError_t launch_stream_select(const IndexerArgs& a, int k, int n_sink, int n_window, Cand* buf, int32_t* buf_n,
                                int cap, hipStream_t stream);

// ---- buckets -----------------------------------------------------------------------------------------------------
struct BucketBuildPlan {
  int64_t chunk;      // positions per scatter chunk
  int64_t n_chunks;
};
BucketBuildPlan bucket_build_plan(int64_t L, int32_t n_buckets);
hipError_t launch_bucket_build(const void* k, int k_dtype, int64_t k_ld, int64_t L, int d, const int32_t* assign,
                               int n_buckets, float* reps, int32_t* offsets, int32_t* members, int32_t* counts,
                               int32_t* table, const BucketBuildPlan& plan, hipStream_t stream);

int bucket_expand_max();
// The no-allocation bucket search keeps its keys in a static device array of bucket_scratch_words() words;
// bucket_scratch returns that array's address on the device of `stream` (looked up once per device).
int64_t bucket_scratch_words();
hipError_t bucket_scratch(hipStream_t stream, uint32_t** out);
// Workspace of the Flat search: keys [B * n_buckets] (uint32, in a Cand-sized area), n_chosen [B],
// gather [B * n_buckets], chosen [B * top_b].
// The Flat search's two steps on their own: slot keys of every bucket (0 for empty ones), then the choice of the
// top_b non-zero slots and their expansion.
hipError_t launch_bucket_scores(const void* q, int q_dtype, int B, int d, const float* reps, const int32_t* offsets,
                                int nb, uint32_t* keys, hipStream_t stream);
hipError_t launch_bucket_choose(const uint32_t* keys, int B, int nb, int top_b, int32_t* buckets_out,
                                const int32_t* offsets, const int32_t* members, int64_t L, const int32_t* t,
                                int n_sink, int n_window, int32_t* idx, int cap, int32_t* n_sel, hipStream_t stream);
// Tree search one level down: the children of each query's kept nodes get their slot keys in keys [B, n_next]
// (bit-identical to launch_bucket_scores for the same representative); other slots are left as they are.
hipError_t launch_tree_children(const void* q, int q_dtype, int B, int d, const int32_t* kept, int keep_ld,
                                const int32_t* n_kept, const int32_t* child_off, const float* reps,
                                const int32_t* offsets, int n_next, uint32_t* keys, hipStream_t stream);
hipError_t launch_bucket_select(const void* q, int q_dtype, int B, int d, const float* reps, const int32_t* offsets,
                                const int32_t* members, int n_buckets, int64_t L, const int32_t* t, int top_b,
                                int n_sink, int n_window, int32_t* idx, int cap, int32_t* n_sel,
                                int32_t* buckets_out, uint32_t* keys, hipStream_t stream);

// ---- attention ---------------------------------------------------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* kv;
  const void* v;
  int dtype;
  int64_t kv_ld, v_ld, L;
  int B, H, d_qk, d_v;
  const int32_t* t;
  const int32_t* idx;
  int idx_ld;
  const int32_t* n_sel;
  int n_sink, n_window;
  float scale;
  void* out;
  float* lse;
};

struct AttnPlan {
  bool mfma;
  int n_splits;
  int rows_per_split;
};
AttnPlan attn_plan(int B, int H, int d_qk, int d_v, int64_t max_rows, int dtype, bool separate_v);
// Bytes of split partials a plan needs, and an upper bound over every read-set bound <= max_rows.
size_t attn_workspace_bytes(const AttnPlan& p, int B, int H, int d_v);
size_t attn_workspace_bound(int B, int H, int d_qk, int d_v, int64_t max_rows, int dtype);
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t stream);

}  // namespace sa
