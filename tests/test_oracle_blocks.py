"""Pins of the block-granular indexers of the oracle ("long-context attention" lecture: sections "Qwen Sparse
Attention" (micro-blocks of pooled index keys, expansion to raw positions, the unfinished micro-block read directly)
and "MiniMax Sparse Attention" (block max of token scores, per-group selection, the local block always kept)).
Each pin ties the functions to something other than their own formulas: the flat token top-k when a block is one
position, hand-built examples with known answers, brute-force loops, and rank counting."""
import numpy as np
import pytest

from oracle import sa_oracle as O


def _rand(seed, L, H=4, d=8, exact=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d))
    w = rng.standard_normal(H)
    k = rng.standard_normal((L, d))
    if exact:  # bf16-representable keys: a one-position mean is the key itself
        k = np.round(k * 16) / 16
    return q, w, k


# ---------------------------------------------------------------------------------------------------------- QSA
@pytest.mark.parametrize("t", [0, 1, 57, 199])
def test_qsa_one_position_blocks_is_the_flat_topk(t):
    q, w, k = _rand(1, 200)
    pooled = O.qsa_pool(k, 1)
    np.testing.assert_array_equal(pooled, k)
    pos, chosen, _ = O.qsa_select(q, w, pooled, t, 1, 13)
    ref, _, _ = O.select_topk(q, w, k, t, 13, 0, 0)
    np.testing.assert_array_equal(pos, ref)
    np.testing.assert_array_equal(chosen, ref)


def test_qsa_tail_and_expansion_by_hand():
    # one head, w = 1, q = e0; the pooled first coordinate of micro-block m (b = 4) is m-dependent by design:
    # block 1 has mean 4, block 2 mean 2, block 0 mean 1, so with k_blocks = 2 the read set is blocks 1 and 2
    # expanded, then the unfinished block's visible positions 12, 13 (t = 13)
    k = np.zeros((16, 2))
    k[0:4, 0] = [1, 1, 1, 1]
    k[4:8, 0] = [4, 4, 3, 5]
    k[8:12, 0] = [2, 2, 2, 2]
    k[12:16, 0] = [100, 100, 100, 100]    # the unfinished block's keys never enter the ranking
    pooled = O.qsa_pool(k, 4)
    np.testing.assert_array_equal(pooled[:, 0], [1, 4, 2, 100])
    q = np.array([[1.0, 0.0]])
    w = np.array([1.0])
    pos, chosen, sc = O.qsa_select(q, w, pooled, 13, 4, 2)
    np.testing.assert_array_equal(chosen, [1, 2])
    np.testing.assert_array_equal(pos, [4, 5, 6, 7, 8, 9, 10, 11, 12, 13])
    np.testing.assert_array_equal(sc, np.float32([1, 4, 2]))
    # t = 15 completes block 3: it wins and there is no tail
    pos, chosen, _ = O.qsa_select(q, w, pooled, 15, 4, 2)
    np.testing.assert_array_equal(chosen, [1, 3])
    np.testing.assert_array_equal(pos, [4, 5, 6, 7, 12, 13, 14, 15])
    # t = 2: no complete block, the three visible positions only
    pos, chosen, _ = O.qsa_select(q, w, pooled, 2, 4, 2)
    assert chosen.size == 0
    np.testing.assert_array_equal(pos, [0, 1, 2])


def test_qsa_ties_and_rank_counting():
    rng = np.random.default_rng(2)
    q, w, k = _rand(2, 400)
    k[:, :] = np.round(k * 2) / 2                   # coarse keys: many equal pooled scores
    pooled = O.qsa_pool(k, 4)
    pos, chosen, sc = O.qsa_select(q, w, pooled, 397, 4, 20)
    n_complete = 398 // 4
    assert sc.size == n_complete and pos.size == 20 * 4 + (398 - 4 * n_complete)
    s = sc.astype(np.float64)
    for m in range(n_complete):                     # a block is chosen iff fewer than 20 blocks rank above it
        above = np.sum((s > s[m]) | ((s == s[m]) & (np.arange(n_complete) < m)))
        assert (m in chosen) == (above < 20)


# ---------------------------------------------------------------------------------------------------------- MSA
@pytest.mark.parametrize("t", [0, 1, 100, 299])
def test_msa_one_position_blocks_is_local_plus_flat_topk(t):
    # c = 1, one group: the local block is position t itself, the others are the flat top-(k_b - 1) before it
    q, w, k = _rand(3, 300)
    (pos, blocks, _), = O.msa_select(q, w, k, t, 1, 1, 9)
    ref = O.select_topk(q, w, k, t - 1, 8, 0, 0)[0] if t > 0 else np.zeros(0, dtype=np.int64)
    np.testing.assert_array_equal(pos, np.concatenate([ref, [t]]))
    assert blocks[-1] == t


def test_msa_block_max_brute_force_and_groups():
    q, w, k = _rand(4, 1000, H=6)
    t, G, c, kb = 777, 3, 64, 4
    res = O.msa_select(q, w, k, t, G, c, kb)
    assert len(res) == G
    local = t // c
    for g, (pos, blocks, bsc) in enumerate(res):
        qs, ws = q[2 * g:2 * g + 2], w[2 * g:2 * g + 2]
        brute = np.zeros(local)
        for blk in range(local):                    # loop over positions and heads
            best = -np.inf
            for s in range(blk * c, blk * c + c):
                v = sum(ws[j] * max(0.0, float(qs[j] @ k[s])) for j in range(2))
                best = max(best, float(np.float32(v)))
            brute[blk] = best
        np.testing.assert_array_equal(bsc.astype(np.float64), brute)
        order = sorted(range(local), key=lambda b_: (-brute[b_], b_))[:kb - 1]
        np.testing.assert_array_equal(blocks, sorted(order) + [local])
        exp = np.concatenate([np.arange(b_ * c, b_ * c + c) for b_ in sorted(order)] + [np.arange(local * c, t + 1)])
        np.testing.assert_array_equal(pos, exp)


def test_msa_groups_choose_independently():
    # group 1's weights are zero: all its block scores tie at 0 and it takes the lowest blocks; group 0 follows q
    k = np.zeros((64, 2))
    k[40:44, 0] = 5.0                              # block 10 (c = 4) stands out for group 0
    q = np.array([[1.0, 0.0], [1.0, 0.0]])
    w = np.array([1.0, 0.0])
    (p0, b0, _), (p1, b1, _) = O.msa_select(q, w, k, 63, 2, 4, 3)
    np.testing.assert_array_equal(b0, [0, 10, 15])  # block 10, then the lowest of the ties (0), then local 15
    np.testing.assert_array_equal(b1, [0, 1, 15])
    np.testing.assert_array_equal(p1, [0, 1, 2, 3, 4, 5, 6, 7, 60, 61, 62, 63])
