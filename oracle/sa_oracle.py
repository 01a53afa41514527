"""CPU oracle of the retrieval-sparse attention path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module. It shares no code
with the HIP path (long_context_sparse_sa_amd/), and the HIP path never calls it.

Everything is computed in fp64 from the exactly decoded stored values (fp32, bfloat16 and FP8 E4M3 values are all
exact in fp64). Library primitives (matmul, sort) serve as steps; nothing is blocked, fused or reordered beyond
the definitions. Sources, cited by page title and section:

  [LongCat] "LongCat Sparse Attention (LSA) deep-dive" (pinghaoyang.com.cn)
      - section "DSA baseline: how the lightning indexer works": the indexer score equation, the arg-topK equation
        and the sparse-attention equation over the latent rows c_s;
      - section "Mechanism 1: streaming-aware indexing (SI)", sub-section on the budget: the selected set is the
        disjoint union of sink, sliding window and the top-K of the indexer over the remaining positions;
        sub-section on the HFA kernel: partial attentions merge exactly by log-sum-exp rescaling.
  [LCA]     "long-context attention" lecture (tju-yxq.github.io): sections "Qwen Sparse Attention" (QSA) and "MiniMax
            Sparse Attention" (MSA), and the read-budget table of its budget calculator.
  [XH]      news page on the open-sourcing of LSA (x-headline.com, 2026-11-04): key facts and the section on its
            principle (keys clustered into a tree-shaped latent structure; the query scans cluster centres only).
  [LSA-8]   "LSA sparse attention: does it save memory? eight QKV entries" (alphalab.site)
      - section 2: Latent Sparse Attention's four steps (index keys; buckets keeping a representative vector and
        member positions; Flat search over representatives; read the chosen rows plus sink plus window);
      - sections 3-4: the eight-entry worked example (stored/read bytes, attention outputs).

Readings taken where the pages are silent:
  * positions are 0-based; sink = [0, n_sink), window = [t-n_window+1, t], both clipped to [0, t];
  * top-k counts only the sparse part and never includes sink or window positions;
  * ties in the fp32 score go to the lower position; ties in bucket score go to the lower bucket id;
  * the reported indexer score is the fp64 value rounded once to fp32, and selection orders by that fp32 value;
  * the bucket score is q . rep (one head, no ReLU, no weight), computed in fp64 and rounded to fp32;
  * a bucket representative is the fp64 mean of its member keys rounded once to fp32;
  * an empty read set yields o = 0 and lse = -inf.

Every function below is pinned by tests under tests/ (test_oracle_*.py) to something other than itself: the
pages' printed eight-entry example, brute force on tiny inputs, closed forms, or a library routine on a special
case. The two whole-step compositions (dsa_step, bucket_step) are pinned by routing the eight-entry example
through them.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------------------------------
# Storage decoding (format definitions: IEEE-754 binary32; bfloat16 = the upper 16 bits of binary32;
# OCP 8-bit floating point E4M3 "fn": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
# exponent field 0, no infinities, S.1111.111 is NaN).
# ----------------------------------------------------------------------------------------------------------------


def decode_f32(raw: np.ndarray) -> np.ndarray:
    return np.asarray(raw, dtype=np.uint32).view(np.float32).astype(np.float64)


def decode_bf16(raw: np.ndarray) -> np.ndarray:
    u = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def decode_e4m3(raw: np.ndarray) -> np.ndarray:
    u = np.asarray(raw, dtype=np.uint8).astype(np.int64)
    sign = np.where((u >> 7) & 1, -1.0, 1.0)
    exp_field = (u >> 3) & 0xF
    mant = (u & 0x7).astype(np.float64)
    normal = (1.0 + mant / 8.0) * np.exp2(exp_field.astype(np.float64) - 7.0)
    subnormal = (mant / 8.0) * np.exp2(-6.0)
    val = sign * np.where(exp_field == 0, subnormal, normal)
    return np.where((exp_field == 0xF) & ((u & 0x7) == 0x7), np.nan, val)


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    return {"f32": decode_f32, "bf16": decode_bf16, "e4m3": decode_e4m3}[dtype](raw)


# ----------------------------------------------------------------------------------------------------------------
# Position sets ([LongCat] SI section, budget equations; 0-based)
# ----------------------------------------------------------------------------------------------------------------


def sink_positions(t: int, n_sink: int) -> np.ndarray:
    return np.arange(0, min(n_sink, t + 1), dtype=np.int64)


def window_positions(t: int, n_window: int) -> np.ndarray:
    return np.arange(max(0, t - n_window + 1), t + 1, dtype=np.int64)


def candidate_positions(t: int, n_sink: int, n_window: int) -> np.ndarray:
    """Positions the indexer ranks: [0, t] minus sink minus window."""
    s = np.arange(0, t + 1, dtype=np.int64)
    fixed = np.union1d(sink_positions(t, n_sink), window_positions(t, n_window))
    return np.setdiff1d(s, fixed, assume_unique=True)


def read_set(t: int, n_sink: int, n_window: int, sparse) -> np.ndarray:
    """R = sink U window U sparse, sorted ascending."""
    fixed = np.union1d(sink_positions(t, n_sink), window_positions(t, n_window))
    return np.union1d(fixed, np.asarray(sparse, dtype=np.int64))


# ----------------------------------------------------------------------------------------------------------------
# Step a1: the lightning indexer ([LongCat] DSA baseline section, indexer equation)
#   I_{t,s} = sum_j w_{t,j} * ReLU(q_{t,j} . k_s), one key k_s shared by all heads j.
# ----------------------------------------------------------------------------------------------------------------


def index_score(q: np.ndarray, w: np.ndarray, k: np.ndarray, positions) -> np.ndarray:
    """fp64 scores of one query over `positions`.

    q: [H, d] fp64 (the query's indexer heads), w: [H] fp64, k: [L, d] fp64, positions: int array.
    """
    pos = np.asarray(positions, dtype=np.int64)
    dots = k[pos] @ q.T                      # [n, H]: q_{t,j} . k_s
    relu = np.maximum(dots, 0.0)             # ReLU per head
    return relu @ w                          # sum_j w_{t,j} * ReLU(...)


def index_score_f32(q, w, k, positions) -> np.ndarray:
    """The reported score: the fp64 value rounded once to fp32."""
    return index_score(q, w, k, positions).astype(np.float32)


# ----------------------------------------------------------------------------------------------------------------
# Step a2: top-k with the sink/window budget ([LongCat] DSA baseline section, arg-topK equation; SI section,
# sparse-part equation: the indexer ranks only positions outside sink and window)
# ----------------------------------------------------------------------------------------------------------------


def topk_positions(score32: np.ndarray, positions, k: int) -> np.ndarray:
    """The min(k, n) positions with the largest fp32 score, ties to the lower position, listed ascending."""
    pos = np.asarray(positions, dtype=np.int64)
    s = np.asarray(score32, dtype=np.float32).astype(np.float64)
    order = np.lexsort((pos, -s))            # primary key: score descending; secondary: position ascending
    return np.sort(pos[order[:min(k, pos.size)]])


def kth_score(score32: np.ndarray, positions, k: int) -> float:
    """The fp32 score of the last selected element (the k-th in (score desc, position asc) order)."""
    pos = np.asarray(positions, dtype=np.int64)
    s = np.asarray(score32, dtype=np.float32).astype(np.float64)
    if pos.size == 0:
        return float("nan")
    order = np.lexsort((pos, -s))
    return float(s[order[min(k, pos.size) - 1]])


def select_topk(q, w, k, t: int, k_sparse: int, n_sink: int, n_window: int):
    """S_sparse for one query: returns (ascending positions, fp32 scores of all candidates, candidate positions)."""
    cand = candidate_positions(t, n_sink, n_window)
    sc = index_score_f32(q, w, k, cand)
    return topk_positions(sc, cand, k_sparse), sc, cand


# ----------------------------------------------------------------------------------------------------------------
# Step a0: the bucket directory ([LSA-8] section 2, step 2: a representative vector and member positions)
# ----------------------------------------------------------------------------------------------------------------


def bucket_build(k: np.ndarray, assign: np.ndarray, n_buckets: int):
    """Returns (reps [NB, d] fp32, offsets [NB+1] int64, members [L] int64).

    members lists positions grouped by bucket, ascending inside each bucket (a stable sort by bucket id);
    reps[c] is the fp64 mean of k over bucket c's members rounded once to fp32 (zeros for an empty bucket).
    """
    assign = np.asarray(assign, dtype=np.int64)
    counts = np.bincount(assign, minlength=n_buckets)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    members = np.argsort(assign, kind="stable").astype(np.int64)
    d = k.shape[1]
    sums = np.zeros((n_buckets, d), dtype=np.float64)
    nonempty = np.nonzero(counts)[0]
    if nonempty.size:
        sums[nonempty] = np.add.reduceat(k[members], offsets[nonempty], axis=0)
    reps = np.zeros((n_buckets, d), dtype=np.float64)
    reps[nonempty] = sums[nonempty] / counts[nonempty, None]
    return reps.astype(np.float32), offsets, members


# ----------------------------------------------------------------------------------------------------------------
# Steps a3 + a4: Flat search over the representatives and expansion to member positions
# ([LSA-8] section 2, steps 3-4)
# ----------------------------------------------------------------------------------------------------------------


def bucket_scores_f32(q: np.ndarray, reps32: np.ndarray) -> np.ndarray:
    """q . rep_c for every bucket, fp64 rounded to fp32."""
    return (np.asarray(reps32, dtype=np.float64) @ q).astype(np.float32)


def top_buckets(score32: np.ndarray, offsets: np.ndarray, top_b: int) -> np.ndarray:
    """The top_b non-empty buckets by (score desc, id asc), in that order."""
    counts = np.diff(offsets)
    ids = np.nonzero(counts > 0)[0]
    s = np.asarray(score32, dtype=np.float32).astype(np.float64)[ids]
    order = np.lexsort((ids, -s))
    return ids[order[:min(top_b, ids.size)]]


def bucket_select(q, reps32, offsets, members, t: int, top_b: int, n_sink: int, n_window: int):
    """Returns (ascending sparse positions, chosen bucket ids, bucket scores)."""
    sc = bucket_scores_f32(q, reps32)
    chosen = top_buckets(sc, offsets, top_b)
    if chosen.size:
        pos = np.concatenate([members[offsets[c]:offsets[c + 1]] for c in chosen])
    else:
        pos = np.zeros(0, dtype=np.int64)
    pos = pos[pos <= t]
    fixed = np.union1d(sink_positions(t, n_sink), window_positions(t, n_window))
    pos = np.setdiff1d(pos, fixed)
    return np.sort(pos), chosen, sc


def tree_select(q, levels, reps32, offsets, members, t: int, keeps, top_b: int, n_sink: int, n_window: int):
    """Tree search over buckets ([LSA-8] section 2, step 3: the Tree variant searches level by level, keeping
    candidates as it goes; [XH] principle section: hierarchical clustering, the query scans cluster centres only).

    Readings where the pages are silent: the tree is an input like the Flat buckets' assignment (its depth and
    fan-out come from the caller's clustering); levels[l] = (reps_l [n_l, d] fp32, child_off_l [n_l + 1]): node i of
    level l has the nodes child_off_l[i] .. child_off_l[i+1]-1 of the next level as children (the last internal
    level's children are buckets); a node's representative is the mean of the keys of every position under it,
    rounded once to fp32 (as a bucket's); at level l the query keeps its keeps[l] best candidate nodes that have
    children (q . rep in fp32, ties to the lower id), and their children are the next level's candidates; at the
    bucket level the top_b best non-empty candidate buckets expand as in the Flat search.
    Returns (ascending sparse positions, chosen bucket ids in (score desc, id asc) order, per-level kept ids)."""
    cand = np.arange(np.asarray(levels[0][0]).shape[0], dtype=np.int64)
    kept_levels = []
    for (reps_l, child_off_l), keep in zip(levels, keeps):
        child_off_l = np.asarray(child_off_l, dtype=np.int64)
        sc = bucket_scores_f32(q, reps_l).astype(np.float64)
        ids = cand[np.diff(child_off_l)[cand] > 0]
        kept = np.sort(ids[np.lexsort((ids, -sc[ids]))][:min(keep, ids.size)])
        kept_levels.append(kept)
        cand = (np.concatenate([np.arange(child_off_l[c], child_off_l[c + 1]) for c in kept]).astype(np.int64)
                if kept.size else np.zeros(0, dtype=np.int64))
    sc = bucket_scores_f32(q, reps32)
    counts = np.diff(offsets)
    ids = cand[counts[cand] > 0]
    s64 = sc.astype(np.float64)[ids]
    chosen = ids[np.lexsort((ids, -s64))][:min(top_b, ids.size)]
    pos = (np.concatenate([members[offsets[c]:offsets[c + 1]] for c in chosen]) if chosen.size
           else np.zeros(0, dtype=np.int64))
    pos = pos[pos <= t]
    fixed = np.union1d(sink_positions(t, n_sink), window_positions(t, n_window))
    pos = np.setdiff1d(pos, fixed)
    return np.sort(pos), chosen, kept_levels


# ----------------------------------------------------------------------------------------------------------------
# Step a5: attention over the read set ([LongCat] DSA baseline section, sparse-attention equation over the
# latent rows c_s shared by all query heads; [LSA-8] section 4: score q.k * scale, softmax, weighted V)
# ----------------------------------------------------------------------------------------------------------------


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of H heads over n rows. q [H, d_qk], K [n, d_qk], V [n, d_v] -> (o [H, d_v], lse [H])."""
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf)
    z = scale * (q @ K.T)                      # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    Z = e.sum(axis=1, keepdims=True)
    o = (e @ V) / Z
    lse = (m + np.log(Z))[:, 0]
    return o, lse


def sparse_attn(q, kv, R, scale: float, d_qk: int, d_v: int, v=None):
    """o over the rows R of the latent cache: K = kv[R, :d_qk], V = kv[R, :d_v] (or v[R, :d_v])."""
    R = np.asarray(R, dtype=np.int64)
    K = kv[R, :d_qk]
    V = (v[R, :d_v] if v is not None else kv[R, :d_v])
    return attention(q, K, V, scale)


def merge_lse(parts):
    """Exact merge of partial attentions over disjoint row sets by their log-sum-exp ([LongCat] SI section, HFA).

    parts: list of (o [H, d_v], lse [H]). Returns (o, lse).
    """
    lses = np.stack([p[1] for p in parts])            # [P, H]
    m = lses.max(axis=0)
    finite = np.isfinite(m)
    msafe = np.where(finite, m, 0.0)
    wts = np.where(np.isfinite(lses), np.exp(lses - msafe), 0.0)
    tot = wts.sum(axis=0)
    o = sum(wts[i][:, None] * parts[i][0] for i in range(len(parts)))
    o = np.where(tot[:, None] > 0, o / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    lse = np.where(tot > 0, msafe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, lse


# ----------------------------------------------------------------------------------------------------------------
# One decode/prefill step of the whole path for one query: selection, read set, attention over it
# ----------------------------------------------------------------------------------------------------------------


def dsa_step(q_idx, w, k_idx, q, kv, t: int, k_sparse: int, n_sink: int, n_window: int, scale: float,
             d_qk: int, d_v: int, v=None):
    """Lightning-indexer top-k ([LongCat] DSA baseline section) plus sink and window ([LongCat] SI section), then
    attention over the read set. Returns (ascending sparse positions, o [H, d_v], lse [H])."""
    sel, _, _ = select_topk(q_idx, w, k_idx, t, k_sparse, n_sink, n_window)
    R = read_set(t, n_sink, n_window, sel)
    o, lse = sparse_attn(q, kv, R, scale, d_qk, d_v, v=v)
    return sel, o, lse


def bucket_step(q_idx, reps32, offsets, members, q, kv, t: int, top_b: int, n_sink: int, n_window: int,
                scale: float, d_qk: int, d_v: int, v=None):
    """Flat bucket search and expansion ([LSA-8] section 2, steps 3-4) plus sink and window, then attention over
    the read set. Returns (ascending sparse positions, chosen bucket ids, o [H, d_v], lse [H])."""
    sel, chosen, _ = bucket_select(q_idx, reps32, offsets, members, t, top_b, n_sink, n_window)
    R = read_set(t, n_sink, n_window, sel)
    o, lse = sparse_attn(q, kv, R, scale, d_qk, d_v, v=v)
    return sel, chosen, o, lse


# ----------------------------------------------------------------------------------------------------------------
# Hierarchical indexing, coarse to fine ([LongCat] section "Mechanism 3: hierarchical indexing (HI)": the cache is
# cut into pages of P positions and each page into sub-blocks of B positions; each sub-block keeps the per-dimension
# mean of its index keys; a page scores the indexer equation summed over its sub-blocks' mean keys; the M best pages
# are recalled and the token-level top-k runs over their positions only).
# Readings where the section is silent:
#   * the mean of a sub-block is over its cached positions (the last one may be partial), computed in fp64 and
#     stored in bf16, the dtype the keys are scored in (rounded to nearest even through fp32, see round_bf16);
#   * query t sees the pages whose first position is <= t; a page's score sums over all its sub-blocks as cached;
#   * pages are ranked by (fp32 page score desc, page id asc); the token stage ranks the sink/window-budget
#     candidates inside the recalled pages exactly like the flat selection.
# ----------------------------------------------------------------------------------------------------------------


def round_bf16(x: np.ndarray) -> np.ndarray:
    """The stored value of an fp64 mean: rounded to fp32 (nearest even), then to bf16 (nearest even on the upper 16
    bits), returned as fp64. This equals one direct rounding to bf16 except when the fp64 value lies within half an
    fp32 ulp of a bf16 midpoint, which needs member keys whose magnitudes differ by more than 2^24."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def hi_means(k: np.ndarray, B: int) -> np.ndarray:
    """Sub-block mean keys [ceil(L / B), d] (bf16 values as fp64)."""
    L, d = k.shape
    n = (L + B - 1) // B
    out = np.zeros((n, d), dtype=np.float64)
    for i in range(n):
        out[i] = k[i * B:min(L, (i + 1) * B)].mean(axis=0)
    return round_bf16(out)


def hi_page_scores(q: np.ndarray, w: np.ndarray, means: np.ndarray, sub_per_page: int, t: int, P: int):
    """fp32 page scores of one query over its visible pages 0 .. floor(t / P): sum over the page's sub-blocks of
    sum_j w_j ReLU(q_j . mean_n), in fp64, rounded once. Returns (scores32, page ids)."""
    n_pages = t // P + 1
    per_sub = index_score(q, w, means, np.arange(means.shape[0]))      # the indexer equation on each mean key
    sc = np.array([per_sub[p * sub_per_page:(p + 1) * sub_per_page].sum() for p in range(n_pages)])
    return sc.astype(np.float32), np.arange(n_pages, dtype=np.int64)


def hi_select(q, w, k, means, t: int, P: int, B: int, M: int, k_sparse: int, n_sink: int, n_window: int):
    """Two-stage selection of one query. Returns (ascending sparse positions, chosen pages ascending, page scores,
    candidate positions of the token stage, their fp32 scores)."""
    psc, pids = hi_page_scores(q, w, means, P // B, t, P)
    pages = topk_positions(psc, pids, M)
    cand = candidate_positions(t, n_sink, n_window)
    cand = cand[np.isin(cand // P, pages)]
    sc = index_score_f32(q, w, k, cand)
    return topk_positions(sc, cand, k_sparse), pages, psc, cand, sc


def hi_step(q_idx, w, k_idx, means, q, kv, t: int, P: int, B: int, M: int, k_sparse: int, n_sink: int,
            n_window: int, scale: float, d_qk: int, d_v: int, v=None):
    """Coarse-to-fine selection ([LongCat] HI section) plus sink and window, then attention over the read set.
    Returns (ascending sparse positions, recalled pages, o [H, d_v], lse [H])."""
    sel, pages, _, _, _ = hi_select(q_idx, w, k_idx, means, t, P, B, M, k_sparse, n_sink, n_window)
    R = read_set(t, n_sink, n_window, sel)
    o, lse = sparse_attn(q, kv, R, scale, d_qk, d_v, v=v)
    return sel, pages, o, lse



# ----------------------------------------------------------------------------------------------------------------
# Block-granular indexers ([LCA] QSA and MSA sections; per-mechanism read budgets in its budget table).
# Readings where the lecture is silent:
#   QSA * a micro-block is b consecutive positions (b = 4 in the release configuration); its pooled index key is
#         the mean of its keys, computed and stored as hi_means does (fp64, rounded through fp32 to bf16);
#       * the normalisation and position encoding the model applies to pooled keys are learned transforms, not
#         part of this path: a caller applies them to the pooled keys before selecting;
#       * a micro-block enters the ranking once all its positions are <= t; it scores the indexer equation on its
#         pooled key; the k_blocks best (fp32 score desc, block id asc) expand to their b positions;
#       * the visible positions of the unfinished micro-block (t+1 mod b of them) are read directly;
#       * the release budget of 2048 tokens is k_blocks = 2048 / b micro-blocks.
#   MSA * the indexer heads form G equal groups (one per GQA group; a group's query heads share its selection);
#         group g's token score is the indexer equation over its own heads, one index key per position;
#       * a block is c consecutive positions (c = 128); its score is the largest visible token score in it;
#       * the block holding t (the local block) is always read; the k_b - 1 best earlier blocks (fp32 score
#         desc, block id asc) complete the group's k_b blocks (16 x 128 = 2048 positions, the table's per-group
#         budget); the local block is read only up to t.
# ----------------------------------------------------------------------------------------------------------------


def qsa_pool(k: np.ndarray, b: int) -> np.ndarray:
    """Pooled index keys of the micro-blocks of b positions (bf16 values as fp64); the last may be partial."""
    return hi_means(k, b)


def qsa_select(q, w, pooled, t: int, b: int, k_blocks: int):
    """QSA read set of one query. Returns (ascending positions: chosen micro-blocks expanded, then the tail;
    chosen block ids ascending; fp32 scores of the complete blocks)."""
    n_complete = (t + 1) // b
    blocks = np.arange(n_complete, dtype=np.int64)
    sc = index_score_f32(q, w, pooled, blocks)
    chosen = topk_positions(sc, blocks, k_blocks)
    expanded = (chosen[:, None] * b + np.arange(b, dtype=np.int64)[None, :]).reshape(-1)
    tail = np.arange(n_complete * b, t + 1, dtype=np.int64)
    return np.concatenate([expanded, tail]), chosen, sc


def msa_block_scores(q, w, k, t: int, G: int, c: int):
    """Per group g: fp32 block scores of the blocks before the local block (max of their token scores)."""
    H = q.shape[0]
    hg = H // G
    local = t // c
    out = []
    for g in range(G):
        tok = index_score_f32(q[g * hg:(g + 1) * hg], w[g * hg:(g + 1) * hg], k, np.arange(local * c))
        out.append(tok.reshape(local, c).max(axis=1) if local > 0 else np.zeros(0, dtype=np.float32))
    return out


def msa_select(q, w, k, t: int, G: int, c: int, k_b: int):
    """MSA read sets of one query, one per group. Returns a list over groups of (ascending positions, chosen block
    ids ascending with the local block last, fp32 block scores of the earlier blocks)."""
    local = t // c
    res = []
    for bsc in msa_block_scores(q, w, k, t, G, c):
        chosen = topk_positions(bsc, np.arange(local, dtype=np.int64), k_b - 1)
        blocks = np.concatenate([chosen, [local]]).astype(np.int64)
        pos = np.concatenate([(chosen[:, None] * c + np.arange(c)[None, :]).reshape(-1),
                              np.arange(local * c, t + 1)]).astype(np.int64)
        res.append((pos, blocks, bsc))
    return res
