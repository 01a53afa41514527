/*
 * sa.h -- C ABI of the retrieval-sparse attention hot path for AMD MI355X (gfx950).
 *
 * The path has three steps, each a call below:
 *   score   an indexer scores every cached position           (sa_index_score, inside sa_select_topk)
 *   select  exact top-k plus sink/window positions             (sa_select_topk; sa_bucket_select and
 *                                                               sa_bucket_tree_select for buckets;
 *                                                               sa_hi_select for the coarse-to-fine search;
 *                                                               sa_qsa_select / sa_msa_select for blocks)
 *   attend  softmax attention over only the gathered rows      (sa_sparse_attn)
 *
 * Sources (web pages; cited by title and section):
 *   [LongCat]  "LongCat Sparse Attention (LSA) deep-dive" (pinghaoyang.com.cn): section "DSA baseline: how the
 *              lightning indexer works" (indexer equation I_{t,s}, arg-topK equation, sparse-attention equation);
 *              section "Mechanism 1: streaming-aware indexing (SI)" (budget decomposition equations; HFA kernel);
 *              section "Mechanism 3: hierarchical indexing (HI)" (sub-block mean keys, page scores, top-M pages,
 *              token top-k inside them).
 *   [LCA]      "long-context attention" lecture (tju-yxq.github.io): sections "Qwen Sparse Attention" (QSA: index keys
 *              pooled over micro-blocks, micro-blocks expanded to raw positions, the unfinished micro-block read
 *              directly) and "MiniMax Sparse Attention" (MSA: block max of token scores, per-group top-k blocks, the
 *              local block always kept); the per-mechanism read budgets of its budget table.
 *   [XH]       news page on the open-sourcing of LSA (x-headline.com, 2026-11-04): key facts and principle section
 *              (keys clustered into a tree; the query scans cluster centres only).
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
 *   - The library keeps no state between calls (apart from the optional, thread-local instrumentation list at the
 *     end of this header) and is thread-safe. Calls on different streams may overlap, provided they share no
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
  SA_TOPK_RADIX_LEVELS = 4, /* few queries over long caches: the radix select over a prefix of the
                             * positions (at most half of them and at most 2^24 keys over all queries), then
                             * key ranges in which only keys above the prefix's k-th key are kept, merged  */
  SA_TOPK_STREAM = 5       /* few queries: scores stay on chip; each launch over a range of positions derives a
                            * proven lower bound of every query's k-th key from per-chunk statistics and emits
                            * only the keys at or above it; one exact merge                                  */
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
 * SA_TOPK_STREAM, SA_TOPK_SPLIT_L and SA_TOPK_PER_QUERY never write the full score matrix (only candidates that
 * can still enter the top-k leave the kernels); SA_TOPK_RADIX writes one 4-byte key per position and query to the
 * workspace, and SA_TOPK_RADIX_LEVELS does so for the positions of its prefix only. SA_TOPK_AUTO takes PER_QUERY
 * for B >= 64 and STREAM below, when the MFMA scorer serves the shape (d = 128, H in {32, 64}, bf16 or e4m3);
 * otherwise RADIX while B * L <= 2^24 and RADIX_LEVELS beyond. SA_TOPK_STREAM's launches wait, for a bounded
 * number of polls, for one another's workgroups (which are sized to be resident together); whatever they see, the
 * bound they use is a proven one, so the result never depends on the timing.
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
 * sa_select_topk_scores -- the selection step of sa_select_topk on caller-given fp32 scores ([LongCat] DSA
 * baseline section, arg-topK equation; SI section, sparse-part equation). It is the test mode of the selection
 * (adversarial score patterns: signed zeros, subnormals, infinities, long runs of equal scores) and serves any
 * caller whose scores come from elsewhere:
 *     S_sparse,b = the min(k_sparse, |C_b|) positions s of C_b with the largest scores[b, s], ties to the LOWER s,
 * where scores compare as fp32 values (-0 == +0; -inf is a valid score). Entries outside C_b are never read as
 * candidates. NaN scores are outside the contract.
 *   scores [B, scores_ld] fp32, scores_ld >= L, 16-byte aligned.      t [B] or NULL (t_b = L - 1).
 *   idx    [B, idx_ld] int32 out, idx_ld >= k_sparse: ascending positions, then -1.   n_sel [B] int32 out.
 *   1 <= k_sparse <= 16384; n_sink, n_window >= 0; L < 2^31.
 *   ws / ws_bytes: at least sa_select_topk_scores_workspace(L, B) bytes (one key per position and query: this
 *   call is given the full score matrix, so keeping its keys costs no more than the input).
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_select_topk_scores_workspace(int64_t L, int32_t B);
SA_API int sa_select_topk_scores(const float* scores, int64_t scores_ld, int64_t L, int32_t B, const int32_t* t,
                                 int32_t k_sparse, int32_t n_sink, int32_t n_window, int32_t* idx, int32_t idx_ld,
                                 int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

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
 * sa_bucket_select_noalloc -- for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): sa_bucket_select with the same arguments minus the workspace,
 * and the same result. Its scratch (one 4-byte key per (query, bucket)) lives in a static device array of the
 * library instead of a caller workspace.
 *   Limit: B * n_buckets <= sa_bucket_select_noalloc_max_keys() (2^21 keys, 8 MiB); a larger call returns
 *   SA_ERR_WORKSPACE and launches nothing.
 *   The array exists once per device, from when the library's device code is loaded there until the process
 *   ends; the first call on a device looks its address up (hipGetSymbolAddress, with that device made current
 *   for the lookup). No call allocates or frees memory.
 *   Every call on one device shares that device's array and leaves its keys behind: calls that may overlap on one
 *   device (different streams, or several host threads) race, and the caller must order them. Nothing in the
 *   array has to start at zero: the kernels write every key they read.
 * ------------------------------------------------------------------------------------------------------------- */
/* ---------------------------------------------------------------------------------------------------------------
 * sa_bucket_tree_select -- Tree bucket search ([LSA-8] section 2, step 3: the Tree variant searches level by level,
 * keeping candidates; [XH] principle section: keys clustered hierarchically, the query scans cluster centres only).
 * The cluster tree is an input, as the Flat buckets' assignment is. Level l (l = 0 .. n_levels-1, root first) has
 * level_n[l] nodes; node i of level l has as children the nodes level_child_off[l][i] .. level_child_off[l][i+1]-1
 * of level l+1 (the buckets for the last level), so siblings are numbered contiguously. A node's representative
 * level_reps[l][i] (fp32 [level_n[l], d]) is the mean of the keys of every position under it (sa_bucket_build with
 * each position assigned to its level-l ancestor writes exactly that). For each query: every root node is scored
 * (q . rep, fp32, as sa_bucket_select scores a bucket, bit-identically), the level_keep[l] best nodes that have
 * children are kept (ties to the lower id), their children are scored, and so on; at the bucket level the top_b
 * best non-empty candidate buckets are chosen and expanded exactly as sa_bucket_select does.
 *   level_reps, level_child_off: HOST arrays of n_levels DEVICE pointers; level_n, level_keep: HOST arrays.
 *   1 <= n_levels <= 8; 1 <= level_keep[l] <= 16384. Child offsets outside the next level are undefined behaviour.
 *   q, reps, offsets, members, n_buckets, L, t, top_b, n_sink, n_window, idx, cap, n_sel, buckets_out: as
 *   sa_bucket_select.
 *   ws / ws_bytes: at least sa_bucket_tree_select_workspace(B, n_levels, level_n, level_keep, n_buckets) bytes.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_bucket_tree_select_workspace(int32_t B, int32_t n_levels, const int32_t* level_n,
                                              const int32_t* level_keep, int32_t n_buckets);
SA_API int sa_bucket_tree_select(const void* q, int q_dtype, int32_t B, int32_t d, int32_t n_levels,
                                 const float* const* level_reps, const int32_t* const* level_child_off,
                                 const int32_t* level_n, const int32_t* level_keep, const float* reps,
                                 const int32_t* offsets, const int32_t* members, int32_t n_buckets, int64_t L,
                                 const int32_t* t, int32_t top_b, int32_t n_sink, int32_t n_window, int32_t* idx,
                                 int32_t cap, int32_t* n_sel, int32_t* buckets_out, void* ws, size_t ws_bytes,
                                 void* stream);

SA_API int64_t sa_bucket_select_noalloc_max_keys(void);
SA_API int sa_bucket_select_noalloc(const void* q, int q_dtype, int32_t B, int32_t d, const float* reps,
                                    const int32_t* offsets, const int32_t* members, int32_t n_buckets, int64_t L,
                                    const int32_t* t, int32_t top_b, int32_t n_sink, int32_t n_window, int32_t* idx,
                                    int32_t cap, int32_t* n_sel, int32_t* buckets_out, void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_hi_build -- the mean keys of the coarse-to-fine index ([LongCat] HI section: every sub-block of B consecutive
 * cached positions keeps the mean of their index keys).
 *   k      [L, k_ld] bf16 index keys (d <= k_ld).
 *   means  [ceil(L / sub_block), d] bf16 out, contiguous: means[n, x] = mean of k[s, x] over the cached positions
 *          s of sub-block n (the last block may be partial); summed in fp64, divided once, rounded to fp32 and
 *          then to bf16, to nearest even both times. Built once per cache (or per appended block); reused by
 *          every sa_hi_select on it.
 *
 * sa_hi_select -- coarse-to-fine top-k ([LongCat] HI section, with the indexer equation of the DSA baseline
 * section applied to the mean keys):
 *   page p (positions [p P, (p+1) P), P = page_len) has score  PS_b(p) = sum over the sub-blocks n of page p of
 *   sum_h w[b,h] relu(q[b,h,:] . means[n,:]), each sub-block term evaluated as sa_index_score evaluates one position
 *   (fp32 accumulation). Query b sees pages whose first position is <= t_b; the n_pages_keep (= M) best visible
 *   pages are recalled (ties: lower page id; fewer if fewer are visible). The token stage then returns the exact
 *   top-k_sparse, as sa_select_topk defines it, of the candidates C_b (outside sink and window) that lie in the
 *   recalled pages.
 *   q, w, k, k_ld, L, B, H, d, t: as sa_index_score; bf16 q and k, d = 128, H in {32, 64}.
 *   means    the output of sa_hi_build for this cache and sub_block.
 *   page_len a multiple of 64 and of sub_block, page_len / sub_block a power of two <= 64.
 *   n_pages_keep in [1, 2^20].  k_sparse in [1, 16384] and <= idx_ld.
 *   idx, idx_ld, n_sel: as sa_select_topk (ascending positions, -1 padding).
 *   pages_out [B, n_pages_keep] int32 or NULL: the recalled pages, ascending, -1 padding.
 *   ws / ws_bytes: at least sa_hi_select_workspace(L, B, sub_block, page_len, n_pages_keep, k_sparse) bytes.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API int sa_hi_build(const void* k, int k_dtype, int64_t k_ld, int64_t L, int32_t d, int32_t sub_block,
                       void* means, void* stream);
SA_API size_t sa_hi_select_workspace(int64_t L, int32_t B, int32_t sub_block, int32_t page_len, int32_t n_pages_keep,
                                     int32_t k_sparse);
SA_API int sa_hi_select(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                        int64_t L, int32_t B, int32_t H, int32_t d, const int32_t* t, const void* means,
                        int32_t sub_block, int32_t page_len, int32_t n_pages_keep, int32_t k_sparse, int32_t n_sink,
                        int32_t n_window, int32_t* idx, int32_t idx_ld, int32_t* n_sel, int32_t* pages_out,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * sa_qsa_pool -- pooled index keys of micro-blocks of `block` consecutive positions ([LCA] QSA section): the mean
 * of their keys, computed exactly as sa_hi_build computes sub-block means (bf16 out, [ceil(L / block), d]). The
 * learned normalisation and position encoding a model applies to pooled keys are not part of this library: a
 * caller applies them to `pooled` before sa_qsa_select.
 *
 * sa_qsa_select -- micro-block selection ([LCA] QSA section): query b ranks the micro-blocks whose positions are
 * all <= t_b by the indexer equation (as sa_index_score) on their pooled keys, keeps the k_blocks best (ties: lower
 * block), and reads them whole, then the visible positions of its unfinished micro-block ((t_b + 1) mod block of
 * them, read directly).
 *   q [B, H, d] bf16, w [B, H] fp32, pooled [ceil(L / block), d] bf16 contiguous (d a multiple of 8), t as
 *   sa_index_score (positions of the L-position cache).
 *   idx [B, idx_ld] int32 out: ascending positions, -1 padding; idx_ld >= k_blocks * block + block - 1.
 *   n_sel [B] int32 out.   k_blocks in [1, 16384].
 *   ws / ws_bytes: at least sa_qsa_select_workspace(L, B, H, d, block, k_blocks) bytes.
 *
 * sa_msa_select -- per-group block selection ([LCA] MSA section): the H indexer heads form G equal groups; for
 * (query b, group g) the token score is the indexer equation over the group's heads, a block of `block` positions
 * scores the largest token score in it, the block holding t_b (the local block) is always read, and the
 * k_blocks - 1 best earlier blocks (ties: lower block) complete the group's blocks.
 *   q, w, k, k_ld, L, B, H, d, t: as sa_index_score; d = 128, H / G in {32, 64}, bf16 or e4m3.
 *   block a multiple of 64.   k_blocks in [1, 16385].
 *   idx [B * G, idx_ld] int32 out (row b * G + g): ascending positions (chosen blocks whole, then the local block up
 *   to t_b), -1 padding; idx_ld >= k_blocks * block.   n_sel [B * G] int32 out.
 *   ws / ws_bytes: at least sa_msa_select_workspace(L, B, G, block, k_blocks) bytes.
 *   For the attention step, row b * G + g is a query whose heads are group g's query heads (sa_sparse_attn with
 *   B * G queries of H_q / G heads each).
 * ------------------------------------------------------------------------------------------------------------- */
SA_API int sa_qsa_pool(const void* k, int k_dtype, int64_t k_ld, int64_t L, int32_t d, int32_t block, void* pooled,
                       void* stream);
SA_API size_t sa_qsa_select_workspace(int64_t L, int32_t B, int32_t H, int32_t d, int32_t block, int32_t k_blocks);
SA_API int sa_qsa_select(const void* q, int q_dtype, const float* w, const void* pooled, int64_t L, int32_t B,
                         int32_t H, int32_t d, const int32_t* t, int32_t block, int32_t k_blocks, int32_t* idx,
                         int32_t idx_ld, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);
SA_API size_t sa_msa_select_workspace(int64_t L, int32_t B, int32_t G, int32_t block, int32_t k_blocks);
SA_API int sa_msa_select(const void* q, int q_dtype, const float* w, const void* k, int k_dtype, int64_t k_ld,
                         int64_t L, int32_t B, int32_t H, int32_t d, int32_t G, const int32_t* t, int32_t block,
                         int32_t k_blocks, int32_t* idx, int32_t idx_ld, int32_t* n_sel, void* ws, size_t ws_bytes,
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
 *   Precision: softmax and accumulation in fp32. When a query's rows are split over several workgroups (few
 *   queries), each split's partial row is kept in the workspace in fp16 after an exact power-of-two scaling per
 *   (head, half of the value columns) that brings it into [-1, 1]; this adds at most 2^-12 of that partial's
 *   largest |value| to each element before the exact merge.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API size_t sa_sparse_attn_workspace(int32_t B, int32_t H, int32_t d_qk, int32_t d_v, int64_t max_rows,
                                       int dtype);
SA_API int sa_sparse_attn(const void* q, const void* kv, const void* v, int dtype, int64_t kv_ld, int64_t v_ld,
                          int64_t L, int32_t B, int32_t H, int32_t d_qk, int32_t d_v, const int32_t* t,
                          const int32_t* idx, int32_t idx_ld, const int32_t* n_sel, int32_t n_sink,
                          int32_t n_window, float scale, void* out, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------------------------------------------
 * Instrumentation (not part of the method): per-kernel timing of the calls above.
 * sa_set_stage_events -- while a list is set on the calling thread, the library records events[i] (a hipEvent_t
 *   created by the caller, passed as void*) on the call's stream right after its i-th kernel launch counted from
 *   this call, for i < n; later launches record nothing. The array (host memory) and the events stay owned by the
 *   caller and must stay valid while the list is set. sa_set_stage_events(NULL, 0) clears the list.
 * sa_stage_events_used -- how many events of the current list have been recorded so far.
 * sa_set_stream_spin_limit -- test knob of SA_TOPK_STREAM on the calling thread: how many times a workgroup polls
 *   for the other workgroups' statistics before it goes on without them (negative: the library's default). A
 *   small limit only makes the bound weaker and the merge larger; the result is the same.
 * ------------------------------------------------------------------------------------------------------------- */
SA_API void sa_set_stage_events(void* const* events, int n);
SA_API int sa_stage_events_used(void);
SA_API void sa_set_stream_spin_limit(int polls);

#ifdef __cplusplus
}
#endif

#endif /* SA_H */
