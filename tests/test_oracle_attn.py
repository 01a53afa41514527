"""Pins of the attention step (LongCat deep-dive, DSA baseline section, sparse-attention equation; SI section,
HFA merge by log-sum-exp): closed forms, invariants, and the reduction to dense softmax attention, which torch's
fp64 CPU scaled_dot_product_attention computes independently.
"""
import numpy as np
import pytest
import torch

from oracle import sa_oracle as O


def test_dense_reduction_matches_library_sdpa():
    """k >= |C|: the read set is every visible position and the result is plain softmax attention."""
    rng = np.random.default_rng(0)
    L, H, d_qk, d_v, Hi, di = 200, 8, 48, 40, 3, 16
    kv = rng.normal(size=(L, 48))
    q = rng.normal(size=(H, d_qk))
    q_idx, w, k_idx = rng.normal(size=(Hi, di)), rng.normal(size=Hi), rng.normal(size=(L, di))
    t = 150
    sel, o, lse = O.dsa_step(q_idx, w, k_idx, q, kv, t, 10_000, 4, 16, 0.125, d_qk, d_v)
    assert O.read_set(t, 4, 16, sel).tolist() == list(range(t + 1))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None, :, None, :], torch.tensor(kv[:t + 1, :d_qk])[None, None].expand(1, H, -1, -1),
        torch.tensor(kv[:t + 1, :d_v])[None, None].expand(1, H, -1, -1), scale=0.125)[0, :, 0, :].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    z = 0.125 * q @ kv[:t + 1, :d_qk].T
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-13)


def test_single_row_returns_that_value_row():
    rng = np.random.default_rng(1)
    kv = rng.normal(size=(10, 6))
    o, lse = O.sparse_attn(rng.normal(size=(3, 6)), kv, [7], 0.3, 6, 6)
    np.testing.assert_array_equal(o, np.repeat(kv[7:8], 3, axis=0))


def test_zero_query_gives_mean_and_log_n():
    rng = np.random.default_rng(2)
    kv = rng.normal(size=(30, 5))
    R = [1, 4, 9, 22]
    o, lse = O.sparse_attn(np.zeros((2, 5)), kv, R, 1.0, 5, 3)
    np.testing.assert_allclose(o, np.repeat(kv[R, :3].mean(axis=0)[None], 2, axis=0), rtol=1e-14)
    np.testing.assert_allclose(lse, np.log(4.0), rtol=1e-15)


def test_separate_v_and_d_v_prefix():
    rng = np.random.default_rng(3)
    kv, v = rng.normal(size=(20, 8)), rng.normal(size=(20, 4))
    q = rng.normal(size=(2, 8))
    o1, _ = O.sparse_attn(q, kv, [0, 5, 6], 0.5, 8, 4, v=v)
    o2, _ = O.attention(q, kv[[0, 5, 6]], v[[0, 5, 6]], 0.5)
    np.testing.assert_array_equal(o1, o2)
    o3, _ = O.sparse_attn(q, kv, [0, 5, 6], 0.5, 8, 4)          # shared latent: V = first d_v columns
    o4, _ = O.attention(q, kv[[0, 5, 6]], kv[[0, 5, 6], :4], 0.5)
    np.testing.assert_array_equal(o3, o4)


@pytest.mark.parametrize("seed", range(4))
def test_lse_merge_invariance(seed):
    rng = np.random.default_rng(seed)
    K, V, q = rng.normal(size=(90, 12)), rng.normal(size=(90, 7)), 3 * rng.normal(size=(4, 12))
    full = O.attention(q, K, V, 0.4)
    cuts = sorted(rng.choice(np.arange(1, 90), size=3, replace=False))
    parts = [O.attention(q, K[a:b], V[a:b], 0.4) for a, b in zip([0] + cuts, cuts + [90])]
    parts.append(O.attention(q, K[:0], V[:0], 0.4))              # an empty part changes nothing
    o, lse = O.merge_lse(parts)
    np.testing.assert_allclose(o, full[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, full[1], rtol=1e-13)


def test_row_order_invariance():
    rng = np.random.default_rng(5)
    K, V, q = rng.normal(size=(40, 9)), rng.normal(size=(40, 9)), rng.normal(size=(3, 9))
    p = rng.permutation(40)
    a, b = O.attention(q, K, V, 0.2), O.attention(q, K[p], V[p], 0.2)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13)


def test_empty_read_set():
    o, lse = O.sparse_attn(np.ones((2, 4)), np.ones((5, 4)), [], 1.0, 4, 4)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
