"""Pins of the hierarchical (coarse-to-fine) indexer of the oracle (LongCat deep-dive, section "Mechanism 3:
hierarchical indexing (HI)": sub-block mean keys, page scores summed over sub-blocks, top-M pages, token top-k
inside them). Each pin ties it to something other than its own formula: the flat selection when every page is
recalled, sums of token scores when a sub-block is one token, closed-form means, and a hand-built example."""
import numpy as np
import pytest

from oracle import sa_oracle as O


def _rand(seed, L, H=3, d=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d))
    w = rng.standard_normal(H)
    k = rng.standard_normal((L, d))
    return q, w, k


def test_means_closed_forms():
    # constant keys: every mean is the constant; a ramp: the mean of s over a block is its midpoint
    k = np.full((37, 4), 0.375)
    np.testing.assert_array_equal(O.hi_means(k, 8), np.full((5, 4), 0.375))
    ramp = np.arange(32, dtype=np.float64)[:, None] * np.ones((1, 2))
    np.testing.assert_array_equal(O.hi_means(ramp, 8)[:, 0], [3.5, 11.5, 19.5, 27.5])
    # a partial last sub-block averages only its cached positions
    np.testing.assert_array_equal(O.hi_means(ramp[:27], 8)[:, 0], [3.5, 11.5, 19.5, 25.0])
    # the stored mean is rounded to nearest-even bf16: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> 1
    x = np.array([[1.0], [1.0 + 2.0 ** -7]])
    assert O.hi_means(x, 2)[0, 0] == 1.0
    x = np.array([[1.0 + 2.0 ** -7], [1.0 + 2.0 ** -6]])     # 1 + 3 * 2^-8: tie between 1+2^-7 and 1+2^-6 -> even
    assert O.hi_means(x, 2)[0, 0] == 1.0 + 2.0 ** -6


def test_every_page_recalled_is_the_flat_selection():
    # M >= the number of visible pages: the token stage ranks every candidate, so HI equals the flat top-k
    for seed, t in [(0, 999), (1, 517), (2, 130)]:
        q, w, k = _rand(seed, 1000)
        means = O.hi_means(k, 4)
        sel, pages, *_ = O.hi_select(q, w, k, means, t, 32, 4, 10_000, 50, 3, 20)
        ref, _, _ = O.select_topk(q, w, k, t, 50, 3, 20)
        np.testing.assert_array_equal(sel, ref)
        assert pages.tolist() == list(range(t // 32 + 1))


def test_one_token_sub_blocks_sum_token_scores():
    # B = 1: each mean key is the key itself (exactly, for bf16-representable keys), so a page's score is the sum
    # of its positions' indexer scores
    rng = np.random.default_rng(3)
    k = np.round(rng.standard_normal((256, 8)) * 8) / 8          # bf16-exact values
    q, w, _ = _rand(3, 1)
    means = O.hi_means(k, 1)
    np.testing.assert_array_equal(means, k)
    psc, pids = O.hi_page_scores(q, w, means, 16, 255, 16)
    tok = O.index_score(q, w, k, np.arange(256))
    np.testing.assert_allclose(psc, tok.reshape(16, 16).sum(axis=1).astype(np.float32), rtol=0, atol=0)


def test_hand_built_recall():
    # one head, w = 1, q = e0. Page 2 of four pages (P = 8, B = 4) holds keys with large first coordinates, page 0
    # small ones: with M = 1 only page 2's positions can be selected, however large a single key elsewhere is
    # relative to its page's mean; the page scores are the sums of ReLU(mean_0) by hand
    k = np.zeros((32, 2))
    k[16:24, 0] = [3, 3, 3, 3, 1, 1, 1, 1]       # page 2: means 3 and 1 -> page score 4
    k[0:8, 0] = [8, -8, -8, -8, 0, 0, 0, 0]      # page 0: means -6 and 0 -> page score 0 (ReLU)
    k[8:16, 0] = [1, 1, 1, 1, 1, 1, 1, 1]        # page 1: means 1 and 1 -> page score 2
    k[24:32, 0] = [2, 2, 2, 2, -1, -1, -1, -1]   # page 3: means 2 and -1 -> page score 2
    q, w = np.array([[1.0, 0.0]]), np.array([1.0])
    means = O.hi_means(k, 4)
    psc, _ = O.hi_page_scores(q, w, means, 2, 31, 8)
    assert psc.tolist() == [0.0, 2.0, 4.0, 2.0]
    sel, pages, *_ = O.hi_select(q, w, k, means, 31, 8, 4, 1, 3, 0, 0)
    assert pages.tolist() == [2] and sel.tolist() == [16, 17, 18]      # position 0 (score 8) is never recalled
    # M = 2: pages 1 and 3 tie at 2 and the lower page id wins; top-10 of pages 1 and 2 by the token score
    # max(k_s0, 0): the four 3s of page 2, then the six lowest positions among the 1s
    sel, pages, *_ = O.hi_select(q, w, k, means, 31, 8, 4, 2, 10, 0, 0)
    assert pages.tolist() == [1, 2]
    assert sel.tolist() == [8, 9, 10, 11, 12, 13, 16, 17, 18, 19]
    # the page of t is visible, a page starting after t is not
    psc, pids = O.hi_page_scores(q, w, means, 2, 16, 8)
    assert pids.tolist() == [0, 1, 2]


@pytest.mark.parametrize("seed", [4, 5])
def test_recall_limits_candidates_to_pages(seed):
    q, w, k = _rand(seed, 4096, H=4, d=16)
    means = O.hi_means(k, 8)
    sel, pages, psc, cand, sc = O.hi_select(q, w, k, means, 4000, 128, 8, 5, 100, 4, 64)
    assert pages.size == 5 and np.all(np.diff(pages) > 0)
    assert np.all(np.isin(sel // 128, pages)) and np.all(np.isin(sel, cand))
    # the recalled pages are the 5 best page scores (ties to lower ids), checked by brute-force rank counting
    order = sorted(range(psc.size), key=lambda p: (-float(psc[p]), p))
    assert sorted(order[:5]) == pages.tolist()


def test_hi_step_with_every_page_recalled_is_the_dsa_step():
    # the whole-step composition reduces to the flat step when every visible page is recalled
    rng = np.random.default_rng(7)
    q_idx, w, k = _rand(7, 300)
    q = rng.standard_normal((2, 16))
    kv = rng.standard_normal((300, 16))
    means = O.hi_means(k, 4)
    sel, pages, o, lse = O.hi_step(q_idx, w, k, means, q, kv, 250, 16, 4, 1000, 30, 2, 10, 0.25, 16, 8)
    sel2, o2, lse2 = O.dsa_step(q_idx, w, k, q, kv, 250, 30, 2, 10, 0.25, 16, 8)
    np.testing.assert_array_equal(sel, sel2)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    assert pages.tolist() == list(range(250 // 16 + 1))
