"""GPU parity of sa_select_topk_scores (the selection on caller-given fp32 scores) against the oracle's top-k
(LongCat deep-dive, DSA baseline section, arg-topK equation; SI section, the sparse part outside sink and window).

The scores are given, so the selection is fully determined: every case is compared bit-exactly, ties included.
The patterns are the ones an order-preserving integer image of fp32 must get right: signed zeros (equal), subnormals
of both signs, infinities, and long runs of equal scores that cross the radix select's position chunks.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from tests.gpu_helpers import selected

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _check(scores32: np.ndarray, k, n_sink=0, n_window=0, t=None):
    B, L = scores32.shape
    sc = torch.tensor(scores32, device=DEV)
    tt = None if t is None else torch.tensor(t, dtype=torch.int32, device=DEV)
    idx, n_sel = sa.sa_select_topk_scores(sc, k, n_sink, n_window, t=tt)
    torch.cuda.synchronize()
    for b in range(B):
        tb = L - 1 if t is None else t[b]
        cand = O.candidate_positions(tb, n_sink, n_window)
        ref = O.topk_positions(scores32[b, cand], cand, k)
        got = selected(idx[b], int(n_sel[b].item()))
        np.testing.assert_array_equal(got, ref)


def _adversarial(rng, B, L):
    pool = np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45, 1.4e-40, -1.4e-40, 1.17549435e-38,
                     -1.17549435e-38, 3.4e38, -3.4e38, 1.0, -1.0, 2.0, 0.5], dtype=np.float32)
    s = pool[rng.integers(0, pool.size, size=(B, L))]
    # a fraction of ordinary values so that the top-k boundary falls inside the special values
    mask = rng.random((B, L)) < 0.3
    s[mask] = rng.standard_normal(mask.sum()).astype(np.float32)
    return s


@pytest.mark.parametrize("seed", [0, 1])
def test_signed_zeros_subnormals_infinities(seed):
    rng = np.random.default_rng(seed)
    _check(_adversarial(rng, 3, 20000), 2048)


def test_only_zeros_of_both_signs():
    # -0 and +0 compare equal: the lowest positions win, whatever the sign bit
    rng = np.random.default_rng(3)
    s = np.where(rng.random((2, 9000)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    _check(s, 100)
    _check(s, 5000)


def test_equal_runs_across_chunks():
    # one long run of equal scores spanning many position chunks of the radix select, a few larger scores
    # scattered through it: the larger ones first, then the lowest positions of the run
    L = 300_000
    s = np.full((2, L), 0.25, dtype=np.float32)
    s[0, [5, 70_000, 299_999]] = 1.0
    s[1, 150_000:150_010] = -1.0
    _check(s, 2048)
    _check(s, 16384)


def test_subnormal_ladder_exact_order():
    # positive and negative subnormals and the smallest normals in a shuffled ladder: the order is the value
    # order of the bit patterns
    rng = np.random.default_rng(4)
    bits = np.concatenate([np.arange(1, 3000, dtype=np.uint32), 0x80000000 + np.arange(1, 3000, dtype=np.uint32),
                           0x00800000 + np.arange(0, 100, dtype=np.uint32)])
    vals = bits.view(np.float32)
    s = vals[rng.permutation(vals.size)][None, :].copy()
    _check(s, 1000)
    _check(s, 3100)


def test_budget_sink_window_and_short_t():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((4, 5000)).astype(np.float32)
    s[:, :] = np.round(s * 4) / 4  # many exact ties
    _check(s, 300, n_sink=4, n_window=128, t=[4999, 2000, 130, 3])
    _check(s, 6000, n_sink=4, n_window=128, t=[4999, 2000, 130, 3])  # k >= |C|: every candidate


def test_single_query_k_one():
    s = np.array([[3.0, 7.0, 7.0, -1.0, 7.0]], dtype=np.float32)
    _check(s, 1)
    _check(s, 2, n_sink=2)
