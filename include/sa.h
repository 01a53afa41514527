/*
 * sa.h -- C ABI of the retrieval-sparse attention hot path for AMD MI355X (gfx950).
 *
 * The path has three steps, each a call below:
 *   score   an indexer scores every cached position           (sa_index_score, inside sa_select_topk)
 *   select  exact top-k plus sink/window positions             (sa_select_topk; sa_bucket_select for buckets)
 *   attend  softmax attention over only the gathered rows      (sa_sparse_attn)
 *
 * Sources (web pages; cited by title and section):
 *   [LongCat]  "LongCat Sparse Attention (LSA) deep-dive" (pinghaoyang.com.cn): section "DSA baseline: how the
 *              lightning indexer works" (indexer equation I_{t,s}, arg-topK equation, sparse-attention equation);
 *              section "Mechanism 1: streaming-aware indexing (SI)" (budget decomposition equations; HFA kernel).
 *   [LSA-8]    "LSA sparse attention: does it save memory? eight QKV entries" (alphalab.site): section 2 (the four
 *              steps of Latent Sparse Attention: index keys, buckets with a representative and member positions,
 *              Flat search over representatives, read selected rows plus sink plus window); sections 3-4 (the
 *              eight-entry worked example).
 *
 * Conventions shared by every call
 *   - Positions are 0-based. The cache holds L positions. Query b sees positions 0..t_b; t == NULL means t_b = L-1
 *     for every query (decode). Values of t outside [0, L) are undefined behaviour.
 *   - sink_b = [0, min(n_sink, t_b+1)), window_b = [max(0, t_b-n_window+1), t_b]. Candidates for the sparse part
 *     C_b = [0, t_b] minus sink_b minus window_b. The read set is R_b = sink_b U window_b U S_sparse,b
 *     ([LongCat] SI section: the three parts are disjoint; the budget pages index from 1, this ABI from 0).
 *   - All data pointers are DEVICE pointers unless stated otherwise, 16-byte aligned, and rows of 2-D arrays are
 *     laid out with the stated leading dimension (in elements). The library never allocates device memory, never
 *     synchronises the stream, and keeps no pointer after a call returns: every launch is asynchronous on
 *     `stream`, and the caller keeps buffers alive until the stream work has completed.
 *   - Inputs are read-only. Outputs are fully overwritten, padding included.
 *   - Arguments are validated on the host before any launch; a non-zero return means nothing was launched
 *     (except SA_ERR_HIP, which reports a failed launch). sa_last_error() gives a thread-local message.
 *   - Scratch memory ("workspace") is caller-owned device memory of at least the size the matching *_workspace
 *     query returns; the queries are pure host functions. A workspace carries nothing from one call to the next:
 *     its contents on entry do not matter, since the kernels clear whatever they accumulate into.
 *   - The library is stateless and thread-safe. Calls on different streams may overlap, provided they share no
 *     workspace and no output buffer.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 */
#ifndef SA_H
#define SA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_API __attribute__((visibility("default")))

/* Element types of stored tensors. SA_E4M3 is the OCP FP8 E4M3 ("fn": no infinities) format. */
typedef enum { SA_F32 = 0, SA_BF16 = 1, SA_E4M3 = 2 } sa_dtype;

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,        /* a required pointer is NULL                                     */
  SA_ERR_SHAPE = 2,       /* a size or leading dimension is out of range                    */
  SA_ERR_DTYPE = 3,       /* unsupported dtype or dtype combination                         */
  SA_ERR_ALIGN = 4,       /* a pointer or leading dimension breaks the alignment rules      */
  SA_ERR_WORKSPACE = 5,   /* workspace pointer NULL or smaller than the query returned      */
  SA_ERR_UNSUPPORTED = 6, /* valid arguments that the library has no kernel for            */
  SA_ERR_HIP = 7          /* a HIP runtime call failed; sa_last_error() holds its message    */
} sa_status;

/* Algorithm choice for sa_select_topk. Every choice returns the same, exactly defined result. */
typedef enum {
  SA_TOPK_AUTO = 0,      /* the library picks by batch size                                            */
  SA_TOPK_SPLIT_L = 1,   /* few queries: key range split over workgroups, thresholds refined by levels  */
  SA_TOPK_PER_QUERY = 2, /* many queries (prefill chunk): one streaming pass per query group             */
  SA_TOPK_RADIX = 3,     /* few queries: one key per position, radix select spread over workgroups      */
  SA_TOPK_RADIX_LEVELS = 4 /* few queries over long caches: the radix select over a prefix of the
                            * positions (at most half of them and at most 2^24 keys over all queries), then
                            * key ranges in which only keys above the prefix's k-th key are kept, merged  */
} sa_topk_algo;

SA_API const char* sa_status_string(int status);
SA_API const char* sa_last_error(void);
SA_API int sa_version(void);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_index_score -- lightning-indexer scores ([LongCat] DSA baseline section, indexer equation):
 *     scores[b, s - s_begin] = sum_{j<H} w[b,j] * max(0, sum_{x<d} q[b,j,x] * k[s,x])   for s_begin <= s < s_end,
 * and -inf where s > t_b. One index key per position is shared by all H indexer heads; there is no scale.
 *   q      [B, H, d] contiguous, dtype q_dtype          w       [B, H] fp32 contiguous
 *   k      [L, d] with leading dimension k_ld >= d, dtype k_dtype
 *   dtypes (q, k): (F32, F32), (BF16, BF16), (E4M3, E4M3). Products are exact in fp32; sums accumulate in fp32.
 *   scores [B, scores_ld] fp32, scores_ld >= s_end - s_begin; 0 <= s_begin <= s_end <= L.
 *   Alignment: q, k rows (k_ld * element size) and scores 16-byte aligned; d * element size a multiple of 16.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API int sa_index_score(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d, const int32_t* t, int64_t s_begin,
                          int64_t s_end, float* scores, int64_t scores_ld, void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_select_topk -- indexer scores fused with exact top-k selection and the sink/window budget ([LongCat] DSA
 * baseline section, arg-topK equation; SI section, sparse-part equation):
 *     S_sparse,b = the min(k_sparse, |C_b|) positions of C_b with the largest fp32 score I_{b,s}
 * where ties are broken towards the LOWER position. The score is the one sa_index_score defines (fp32).
 * SA_TOPK_SPLIT_L and SA_TOPK_PER_QUERY never write the full score matrix (only candidates that can still enter
 * the top-k leave the kernels); SA_TOPK_RADIX writes one 4-byte key per position and query to the workspace, and
 * SA_TOPK_RADIX_LEVELS does so for the positions of its prefix only. SA_TOPK_AUTO takes PER_QUERY for B >= 64,
 * RADIX while B * L <= 2^24, RADIX_LEVELS beyond.
 *   idx    [B, idx_ld] int32, idx_ld >= k_sparse: S_sparse,b in ascending position order, then -1 padding.
 *   n_sel  [B] int32: |S_sparse,b|.
 *   The sink and window are not listed in idx; pass the same n_sink/n_window to sa_sparse_attn.
 *   k_sparse >= 1, n_sink >= 0, n_window >= 0. L < 2^31.
 *   ws / ws_bytes: workspace of at least sa_select_topk_workspace(L, B, H, d, q_dtype, k_dtype, k_sparse, algo)
 *   bytes. 1 <= k_sparse <= 16384.
 *   algo: an sa_topk_algo value; SA_TOPK_PER_QUERY needs d = 128, H in {32, 64} and bf16 or e4m3 inputs.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_select_topk_workspace(int64_t L, int32_t B, int32_t H, int32_t d, int q_dtype, int k_dtype,
                                       int32_t k_sparse, int algo);
SA_API int sa_select_topk(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d, const int32_t* t, int32_t k_sparse,
                          int32_t n_sink, int32_t n_window, int32_t* idx, int32_t idx_ld, int32_t* n_sel,
                          void* ws, size_t ws_bytes, int algo, void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_bucket_build -- the bucket directory of Latent Sparse Attention ([LSA-8] section 2, step 2: each bucket
 * keeps a representative vector and the positions of its members). Built once per cache.
 *   k        [L, d] index keys, leading dimension k_ld, dtype F32 or BF16
 *   assign   [L] int32 bucket id of each position, in [0, n_buckets)
 *   reps     [n_buckets, d] fp32 out: mean of the member keys (sum in fp64, rounded once to fp32); 0 if empty
 *   offsets  [n_buckets + 1] int32 out: exclusive prefix sum of bucket sizes (CSR)
 *   members  [L] int32 out: positions grouped by bucket, ascending inside each bucket
 *   ws / ws_bytes: at least sa_bucket_build_workspace(L, n_buckets) bytes.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_bucket_build_workspace(int64_t L, int32_t n_buckets);
SA_API int sa_bucket_build(const void* k, int k_dtype, int64_t k_ld, int64_t L, int32_t d, const int32_t* assign,
                           int32_t n_buckets, float* reps, int32_t* offsets, int32_t* members, void* ws,
                           size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_bucket_select -- Flat bucket search and expansion ([LSA-8] section 2, steps 3-4): score every non-empty
 * bucket by the fp32 dot product q_b . rep_c (single head, no ReLU, no weight), keep the top_b buckets (ties to
 * the lower bucket id), expand them to their member positions s <= t_b, drop sink and window positions, and list
 * the result in ascending order.
 *   q        [B, d] dtype F32 or BF16 contiguous; reps/offsets/members as written by sa_bucket_build.
 *   idx      [B, cap] int32 out: ascending positions, -1 padding. n_sel [B] out: count, or -(needed count) when
 *            the expansion does not fit in cap (idx then holds no valid entries for that query).
 *   buckets_out [B, top_b] int32 out or NULL: chosen bucket ids in (score desc, id asc) order, -1 padding.
 *   1 <= top_b <= n_buckets; top_b <= 1024; 1 <= cap <= 16384. assign/offsets/members must be as
 *   sa_bucket_build wrote them (values outside [0, n_buckets) are undefined behaviour).
 *   ws / ws_bytes: at least sa_bucket_select_workspace(B, n_buckets, top_b) bytes.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_bucket_select_workspace(int32_t B, int32_t n_buckets, int32_t top_b);
SA_API int sa_bucket_select(const void* q, int q_dtype, int32_t B, int32_t d, const float* reps,
                            const int32_t* offsets, const int32_t* members, int32_t n_buckets, int64_t L,
                            const int32_t* t, int32_t top_b, int32_t n_sink, int32_t n_window, int32_t* idx,
                            int32_t cap, int32_t* n_sel, int32_t* buckets_out, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_sparse_attn -- attention over the read set only ([LongCat] DSA baseline section, sparse-attention equation,
 * in MLA absorbed-MQA form: one cached latent row per position is shared by every query head):
 *     o[b,h,:] = sum_{s in R_b} softmax_s(scale * q[b,h,:] . K_s) * V_s,   lse[b,h] = log sum_{s in R_b} exp(...)
 * with K_s = kv[s, 0:d_qk] and V_s = kv[s, 0:d_v] (v == NULL, shared latent) or v[s, 0:d_v]. Sink and window rows
 * are contiguous ranges; partial results over disjoint row subsets are merged exactly by their log-sum-exp
 * ([LongCat] SI section, HFA: online-softmax rescaling of the partial outputs).
 *   q    [B, H, d_qk] contiguous, dtype `dtype`     kv [L, kv_ld]     v [L, v_ld] or NULL
 *   d_v <= 1024.
 *   dtype: F32 or BF16 for q, kv, v and out.
 *   idx  [B, idx_ld] int32: sparse positions; only the first clamp(n_sel[b], 0, idx_ld) entries are read. They
 *        must be distinct, inside [0, t_b] and outside sink_b and window_b (as sa_select_topk and
 *        sa_bucket_select write them). idx/n_sel may be NULL together (sink and window only).
 *   out  [B, H, d_v] dtype `dtype`. lse [B, H] fp32 (natural log) or NULL. An empty read set gives o = 0 and
 *        lse = -inf.
 *   ws / ws_bytes: at least sa_sparse_attn_workspace(B, H, d_qk, d_v, max_rows, dtype) bytes, where
 *        max_rows >= n_sink + n_window + idx_ld bounds every read set.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_sparse_attn_workspace(int32_t B, int32_t H, int32_t d_qk, int32_t d_v, int64_t max_rows,
                                       int dtype);
SA_API int sa_sparse_attn(const void* q, const void* kv, const void* v, int dtype, int64_t kv_ld, int64_t v_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d_qk, int32_t d_v, const int32_t* t,
                          const int32_t* idx, int32_t idx_ld, const int32_t* n_sel, int32_t n_sink,
                          int32_t n_window, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
