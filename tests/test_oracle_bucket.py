"""Pins of the bucket directory and the Flat bucket search (LSA eight-entry page, section 2, steps 2-4)."""
import numpy as np
import pytest

from oracle import sa_oracle as O
from tests.test_oracle_select import brute_force_topk


@pytest.mark.parametrize("seed", range(5))
def test_csr_invariants(seed):
    rng = np.random.default_rng(seed)
    L, NB = int(rng.integers(1, 400)), int(rng.integers(1, 40))
    assign = rng.integers(0, NB, size=L)
    k = rng.normal(size=(L, 3))
    reps, offsets, members = O.bucket_build(k, assign, NB)
    assert offsets[0] == 0 and offsets[-1] == L and np.all(np.diff(offsets) >= 0)
    assert sorted(members.tolist()) == list(range(L))
    for c in range(NB):
        seg = members[offsets[c]:offsets[c + 1]]
        assert np.all(assign[seg] == c) and np.all(np.diff(seg) > 0)
        if seg.size:
            np.testing.assert_allclose(reps[c], k[seg].mean(axis=0), rtol=1e-6, atol=1e-7)
        else:
            assert np.all(reps[c] == 0)


def test_rep_closed_form_by_hand():
    k = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 8.0]])
    reps, offsets, members = O.bucket_build(k, np.array([1, 0, 1]), 3)
    assert reps.tolist() == [[3.0, 4.0], [3.0, 5.0], [0.0, 0.0]]
    assert offsets.tolist() == [0, 1, 3, 3] and members.tolist() == [1, 0, 2]


def test_empty_buckets_are_never_chosen():
    reps = np.array([[0.0, 0.0], [1.0, 0.0], [9.0, 0.0]], dtype=np.float32)
    offsets = np.array([0, 2, 4, 4])                 # bucket 2 is empty (but has the best score)
    members = np.array([0, 3, 1, 2])
    sel, chosen, _ = O.bucket_select(np.array([1.0, 0.0]), reps, offsets, members, 3, 2, 0, 0)
    assert chosen.tolist() == [1, 0] and sel.tolist() == [0, 1, 2, 3]


def test_bucket_score_ties_go_to_lower_id():
    reps = np.array([[1.0, 0.0], [2.0, 0.0], [2.0, 0.0]], dtype=np.float32)
    offsets, members = np.array([0, 1, 2, 3]), np.array([0, 1, 2])
    _, chosen, _ = O.bucket_select(np.array([1.0, 0.0]), reps, offsets, members, 2, 1, 0, 0)
    assert chosen.tolist() == [1]


@pytest.mark.parametrize("seed", range(6))
def test_singleton_buckets_reduce_to_plain_topk(seed):
    """With one position per bucket, rep = key and the Flat search is a plain top-k of q.k (no ReLU)."""
    rng = np.random.default_rng(seed)
    L, d, kk = 60, 3, int(rng.integers(1, 30))
    k = rng.integers(-2, 3, size=(L, d)).astype(np.float64)
    q = rng.integers(-2, 3, size=d).astype(np.float64)
    reps, offsets, members = O.bucket_build(k, np.arange(L), L)
    sel, _, _ = O.bucket_select(q, reps, offsets, members, L - 1, kk, 0, 0)
    assert sel.tolist() == brute_force_topk((k @ q).tolist(), list(range(L)), kk)


def test_expansion_drops_future_sink_and_window():
    k = np.zeros((12, 1))
    assign = np.array([0] * 12)
    reps, offsets, members = O.bucket_build(k, assign, 1)
    sel, _, _ = O.bucket_select(np.array([1.0]), reps, offsets, members, 9, 1, 2, 3)
    assert sel.tolist() == [2, 3, 4, 5, 6]           # t=9: drop 10,11 (future), 0,1 (sink), 7,8,9 (window)
