// Internal launch interface between the C ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sa {

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
};

// One emitted candidate: (order-preserving key of the fp32 score, position).
struct Cand {
  uint32_t key;
  int32_t pos;
};

enum ScoreMode { kScoreDense = 0, kScoreEmit = 1, kScoreAll = 2 };

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
// Workspace of the Flat search: keys [B * n_buckets] (uint32, in a Cand-sized area), n_chosen [B],
// gather [B * n_buckets], chosen [B * top_b].
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
