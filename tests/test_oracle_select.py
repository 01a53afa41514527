"""Pins of the indexer score and the top-k selection (LongCat deep-dive: DSA baseline section, indexer and arg-topK
equations; SI section, budget equations).

Integer-valued inputs make every score exact in fp32 and fp64, so selection is checked exactly, ties included,
against a brute-force rank count that shares nothing with the oracle's sort.
"""
import itertools

import numpy as np
import pytest

from oracle import sa_oracle as O


def brute_force_topk(scores, positions, k):
    """Position p is selected iff fewer than k candidates beat it: higher score, or equal score and lower position."""
    sel = []
    for i, p in enumerate(positions):
        beaten_by = sum(1 for j, pj in enumerate(positions)
                        if scores[j] > scores[i] or (scores[j] == scores[i] and pj < p))
        if beaten_by < k:
            sel.append(p)
    return sorted(sel)


def brute_force_score(q, w, k, s):
    total = 0.0
    for j in range(q.shape[0]):
        dot = 0.0
        for x in range(q.shape[1]):
            dot += q[j, x] * k[s, x]
        total += w[j] * (dot if dot > 0 else 0.0)
    return total


def test_candidate_sets_by_hand():
    assert O.candidate_positions(9, 2, 3).tolist() == [2, 3, 4, 5, 6]
    assert O.candidate_positions(3, 2, 3).tolist() == []              # sink {0,1} and window {1,2,3} overlap
    assert O.candidate_positions(5, 0, 0).tolist() == [0, 1, 2, 3, 4, 5]
    assert O.candidate_positions(0, 4, 32).tolist() == []
    assert O.read_set(9, 2, 3, [4, 5]).tolist() == [0, 1, 4, 5, 7, 8, 9]
    assert O.sink_positions(2, 4).tolist() == [0, 1, 2]               # sink clipped to [0, t]
    assert O.window_positions(2, 32).tolist() == [0, 1, 2]


@pytest.mark.parametrize("seed", range(12))
def test_selection_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    L, H, d = int(rng.integers(20, 60)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
    q = rng.integers(-2, 3, size=(H, d)).astype(np.float64)
    w = rng.integers(0, 3, size=H).astype(np.float64)
    k = rng.integers(-2, 3, size=(L, d)).astype(np.float64)
    t = int(rng.integers(0, L))
    n_sink, n_window, kk = int(rng.integers(0, 5)), int(rng.integers(0, 6)), int(rng.integers(1, 25))
    sel, sc, cand = O.select_topk(q, w, k, t, kk, n_sink, n_window)
    bf_scores = [brute_force_score(q, w, k, s) for s in cand]
    np.testing.assert_array_equal(sc, np.array(bf_scores, dtype=np.float32))
    assert sel.tolist() == brute_force_topk(bf_scores, cand.tolist(), kk)
    assert len(sel) == min(kk, len(cand))


def test_all_candidates_when_k_exceeds():
    rng = np.random.default_rng(7)
    q, w, k = rng.normal(size=(2, 4)), rng.uniform(size=2), rng.normal(size=(50, 4))
    sel, _, cand = O.select_topk(q, w, k, 40, 1000, 3, 5)
    assert sel.tolist() == cand.tolist() == [s for s in range(41) if 3 <= s <= 35]


def test_relu_and_weight_sign():
    """w * ReLU(x), not ReLU(w * x): a negative weight subtracts the positive part only."""
    q = np.array([[1.0, -1.0]])
    k = np.array([[2.0, 1.0], [1.0, 2.0]])        # dots: +1 and -1
    assert O.index_score(q, np.array([-3.0]), k, [0, 1]).tolist() == [-3.0, 0.0]
    assert O.index_score(q, np.array([3.0]), k, [0, 1]).tolist() == [3.0, 0.0]


def test_invariant_under_positive_scaling_and_head_permutation():
    rng = np.random.default_rng(3)
    q = rng.integers(-2, 3, size=(5, 3)).astype(np.float64)
    w = rng.integers(-2, 3, size=5).astype(np.float64)
    k = rng.integers(-2, 3, size=(64, 3)).astype(np.float64)
    base, _, _ = O.select_topk(q, w, k, 63, 10, 2, 4)
    s2, _, _ = O.select_topk(q, 4.0 * w, k, 63, 10, 2, 4)
    s3, _, _ = O.select_topk(2.0 * q, w, k, 63, 10, 2, 4)
    perm = rng.permutation(5)
    s4, _, _ = O.select_topk(q[perm], w[perm], k, 63, 10, 2, 4)
    assert base.tolist() == s2.tolist() == s3.tolist() == s4.tolist()


def test_single_head_unit_query_is_relu_of_a_key_column():
    rng = np.random.default_rng(4)
    k = rng.normal(size=(30, 6))
    for col in range(6):
        q = np.zeros((1, 6))
        q[0, col] = 1.0
        np.testing.assert_array_equal(O.index_score(q, np.array([1.0]), k, np.arange(30)), np.maximum(k[:, col], 0))


def test_kth_score():
    sc = np.array([5, 3, 3, 9, 1], dtype=np.float32)
    pos = np.array([0, 1, 2, 3, 4])
    assert O.kth_score(sc, pos, 1) == 9 and O.kth_score(sc, pos, 3) == 3 and O.kth_score(sc, pos, 10) == 1
    assert O.topk_positions(sc, pos, 3).tolist() == [0, 1, 3]


def test_exhaustive_tiny():
    """Every score pattern over 4 candidates with values in {0,1,2} and every k."""
    pos = [3, 5, 6, 9]
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=4):
        for kk in range(1, 6):
            got = O.topk_positions(np.array(vals, dtype=np.float32), np.array(pos), kk).tolist()
            assert got == brute_force_topk(list(vals), pos, kk)
