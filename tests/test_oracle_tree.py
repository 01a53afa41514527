"""Pins of the oracle's Tree bucket search (LSA eight-entry page, section 2, step 3: the Tree variant searches level by
level; news page on the open-sourcing of LSA, principle section: hierarchical clustering, cluster centres scanned).
The pins: keeping every node reduces the Tree to the Flat search; a hand-built two-level tree whose coarse choice
hides the best bucket; the eight-entry worked example under one root; brute force on small random trees."""
import numpy as np
import pytest

from oracle import sa_oracle as O


def _tree(rng, L, d, n_buckets, fan):
    """A random two-level tree: positions -> buckets, buckets numbered so that siblings are contiguous, groups of
    `fan` consecutive buckets under one parent. Returns the level list and the bucket directory."""
    k = rng.standard_normal((L, d))
    assign = rng.integers(0, n_buckets, size=L)
    reps, offsets, members = O.bucket_build(k, assign, n_buckets)
    n_top = (n_buckets + fan - 1) // fan
    parent = np.arange(n_buckets) // fan
    top_reps, top_off, _ = O.bucket_build(k, parent[assign], n_top)
    child_off = np.minimum(np.arange(n_top + 1) * fan, n_buckets)
    # a parent with no positions has a mean of 0 but its children are empty buckets: keep the child ranges
    return k, [(top_reps, child_off)], reps, offsets, members, top_off


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_keeping_every_node_is_the_flat_search(seed):
    rng = np.random.default_rng(seed)
    k, levels, reps, offsets, members, _ = _tree(rng, 3000, 8, 60, 7)
    q = rng.standard_normal(8)
    for t, top_b in [(2999, 5), (1500, 12), (40, 3)]:
        pos, chosen, _ = O.tree_select(q, levels, reps, offsets, members, t, [10_000], top_b, 4, 16)
        ref, ref_chosen, _ = O.bucket_select(q, reps, offsets, members, t, top_b, 4, 16)
        np.testing.assert_array_equal(pos, ref)
        np.testing.assert_array_equal(chosen, ref_chosen)


def test_coarse_choice_hides_the_best_bucket():
    # d = 1, q = 1: bucket score = bucket mean. Parent 0 = buckets {0, 1} with means {5, -5} (parent mean 0);
    # parent 1 = buckets {2, 3} with means {1, 1.5} (parent mean 1.25). Keeping one parent picks parent 1, so bucket 0
    # (the best single bucket) is never seen.
    k = np.array([[5.0], [5.0], [-5.0], [-5.0], [1.0], [1.0], [1.5], [1.5]])
    assign = np.array([0, 0, 1, 1, 2, 2, 3, 3])
    reps, offsets, members = O.bucket_build(k, assign, 4)
    top_reps, _, _ = O.bucket_build(k, np.array([0, 0, 0, 0, 1, 1, 1, 1]), 2)
    np.testing.assert_array_equal(top_reps[:, 0], [0.0, 1.25])
    levels = [(top_reps, np.array([0, 2, 4]))]
    q = np.array([1.0])
    pos, chosen, kept = O.tree_select(q, levels, reps, offsets, members, 7, [1], 1, 0, 0)
    np.testing.assert_array_equal(kept[0], [1])
    np.testing.assert_array_equal(chosen, [3])
    np.testing.assert_array_equal(pos, [6, 7])
    flat, flat_chosen, _ = O.bucket_select(q, reps, offsets, members, 7, 1, 0, 0)
    np.testing.assert_array_equal(flat_chosen, [0])
    np.testing.assert_array_equal(flat, [0, 1])


def test_eight_entry_example_under_one_root():
    # the worked example's buckets A = positions 0-3 and B = 4-7 under a single root: the tree keeps the root and
    # then behaves as the Flat search (A first for q = (1, 0))
    k = np.array([[1, 0], [0.8, 0.2], [0.6, 0.4], [0.4, 0.6], [0, 1], [-0.2, 0.8], [-0.4, 0.6], [-0.6, 0.4]])
    assign = np.array([0, 0, 0, 0, 1, 1, 1, 1])
    reps, offsets, members = O.bucket_build(k, assign, 2)
    root, _, _ = O.bucket_build(k, np.zeros(8, dtype=np.int64), 1)
    pos, chosen, _ = O.tree_select(np.array([1.0, 0.0]), [(root, np.array([0, 2]))], reps, offsets, members, 7,
                                   [1], 1, 0, 0)
    np.testing.assert_array_equal(chosen, [0])
    np.testing.assert_array_equal(pos, [0, 1, 2, 3])


def test_brute_force_two_levels():
    rng = np.random.default_rng(5)
    k, levels, reps, offsets, members, top_off = _tree(rng, 800, 4, 30, 4)
    (top_reps, child_off), = levels
    for trial in range(6):
        q = rng.standard_normal(4)
        t, keep, top_b = int(rng.integers(100, 800)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        pos, chosen, kept = O.tree_select(q, levels, reps, offsets, members, t, [keep], top_b, 2, 5)
        # brute force: explicit loops over nodes with fp32-rounded dot products
        def s32(v):
            return float(np.float32(sum(float(a) * float(b) for a, b in zip(q, v))))
        tops = [i for i in range(len(top_reps)) if child_off[i + 1] > child_off[i]]
        tops.sort(key=lambda i: (-s32(top_reps[i]), i))
        kk = sorted(tops[:keep])
        np.testing.assert_array_equal(kept[0], kk)
        cands = [c for i in kk for c in range(child_off[i], child_off[i + 1]) if offsets[c + 1] > offsets[c]]
        cands.sort(key=lambda c: (-s32(reps[c]), c))
        np.testing.assert_array_equal(chosen, cands[:top_b])
        want = sorted(p for c in cands[:top_b] for p in members[offsets[c]:offsets[c + 1]]
                      if 2 <= p <= t - 5)
        np.testing.assert_array_equal(pos, want)


def test_three_levels_keep_everything_is_flat():
    rng = np.random.default_rng(6)
    k, (lvl1,), reps, offsets, members, top_off = _tree(rng, 2000, 6, 48, 4)     # 12 parents of 4 buckets
    n_mid = lvl1[0].shape[0]
    # a root level over the 12 parents, 3 per root
    parent_of_bucket = np.arange(48) // 4
    root_of_mid = np.arange(n_mid) // 3
    # root representatives: the mean of the keys under each root (via the bucket of each position)
    pos_bucket = np.empty(2000, dtype=np.int64)
    for c in range(48):
        pos_bucket[members[offsets[c]:offsets[c + 1]]] = c
    root_reps, _, _ = O.bucket_build(k, root_of_mid[parent_of_bucket[pos_bucket]], 4)
    levels = [(root_reps, np.minimum(np.arange(5) * 3, n_mid)), lvl1]
    q = rng.standard_normal(6)
    pos, chosen, kept = O.tree_select(q, levels, reps, offsets, members, 1999, [100, 100], 6, 0, 0)
    ref, ref_chosen, _ = O.bucket_select(q, reps, offsets, members, 1999, 6, 0, 0)
    np.testing.assert_array_equal(chosen, ref_chosen)
    np.testing.assert_array_equal(pos, ref)
    assert len(kept) == 2
