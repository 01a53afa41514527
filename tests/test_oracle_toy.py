"""Pins of the oracle to the pages' eight-entry worked example (LSA eight-entry page, sections 3-4).

The page prints the attention outputs to two decimals (36.45 full read, 23.24 bucket A only, second dimension 0)
and the byte accounting (64 B stored, 32 B read, 40 B directory). Derived values come from the same data by hand.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import sa_oracle as O
from sa_workloads import perf


@pytest.fixture(scope="module")
def toy(golden_dir):
    with open(os.path.join(golden_dir, "toy_8entry.json")) as f:
        g = json.load(f)
    K = np.array(g["keys_bucket_A"] + g["keys_bucket_B"], dtype=np.float64)
    V = np.array(g["values"], dtype=np.float64)
    q = np.array(g["q"], dtype=np.float64)
    return g, q, K, V


SCALE = 1.0 / math.sqrt(2.0)


def test_printed_full_and_bucket_a(toy):
    g, q, K, V = toy
    o_full, _ = O.attention(q[None, :], K, V, SCALE)
    o_a, _ = O.attention(q[None, :], K[:4], V[:4], SCALE)
    assert abs(o_full[0, 0] - g["printed"]["attn_dim0_full_read"]) < 0.005
    assert abs(o_a[0, 0] - g["printed"]["attn_dim0_bucket_A_only"]) < 0.005
    assert o_full[0, 1] == g["printed"]["attn_dim1"] and o_a[0, 1] == 0.0
    assert o_full[0, 0] == pytest.approx(g["derived"]["attn_dim0_full_read"], rel=1e-13)
    assert o_a[0, 0] == pytest.approx(g["derived"]["attn_dim0_bucket_A_only"], rel=1e-13)


def test_printed_bytes(toy):
    g, *_ = toy
    p = g["printed"]
    assert perf.stored_bytes(8, 2 + 2, g["bytes_per_number"]) == p["stored_bytes_all_8"]
    assert perf.read_bytes(4, 2 + 2, g["bytes_per_number"]) == p["read_bytes_bucket_A"]
    assert perf.directory_bytes(2, 2, g["bytes_per_number"], 8, g["position_id_bytes"]) == p["directory_bytes"]


def test_kv_calculator(golden_dir):
    with open(os.path.join(golden_dir, "kv_size_calculator.json")) as f:
        g = json.load(f)
    b = perf.kv_cache_bytes_mha(g["layers"], g["H_kv"], g["d"], g["S"], g["bytes"])
    assert b / 2**30 == g["printed_gib"]
    mla = perf.kv_cache_bytes_mla(g["layers"], 512, 64, g["S"], g["bytes"])
    share = 100.0 * mla / perf.kv_cache_bytes_mha(g["layers"], 32, 128, g["S"], g["bytes"])
    assert round(share) == g["printed_mla_share_percent_approx"]


def test_dsa_path_through_toy(toy):
    """One indexer head with w=1 and q_idx=(1,0) over the eight keys reproduces the bucket-A read."""
    g, q, K, V = toy
    sc = O.index_score(q[None, :], np.array([1.0]), K, np.arange(8))
    np.testing.assert_allclose(sc, g["derived"]["dsa_scores_one_head_w1"], rtol=0, atol=1e-15)
    sc2 = O.index_score(np.array([[1.0, 0.0], [0.0, 1.0]]), np.array([1.0, 2.0]), K, np.arange(8))
    np.testing.assert_allclose(sc2, g["derived"]["dsa_scores_two_heads_q10_q01_w1_w2"], rtol=0, atol=1e-15)
    scn = O.index_score(q[None, :], np.array([-1.0]), K, np.arange(8))
    np.testing.assert_allclose(scn, g["derived"]["dsa_scores_one_head_w_minus1"], rtol=0, atol=1e-15)
    # top-4 picks bucket A; top-5 breaks a four-way tie at score 0 towards position 4; top-8 reads everything
    for k, expect_pos, expect_o in [(4, [0, 1, 2, 3], "attn_dim0_bucket_A_only"),
                                    (5, [0, 1, 2, 3, 4], "attn_dim0_positions_0_to_4"),
                                    (8, list(range(8)), "attn_dim0_full_read")]:
        sel, _, _ = O.select_topk(q[None, :], np.array([1.0]), K, 7, k, 0, 0)
        assert sel.tolist() == expect_pos
        o, _ = O.sparse_attn(q[None, :], K, O.read_set(7, 0, 0, sel), SCALE, 2, 2, v=V)
        assert o[0, 0] == pytest.approx(g["derived"][expect_o], rel=1e-13)


def test_bucket_path_through_toy(toy):
    g, q, K, V = toy
    assign = np.array([0, 0, 0, 0, 1, 1, 1, 1])
    reps, offsets, members = O.bucket_build(K, assign, 2)
    np.testing.assert_array_equal(reps, np.array([g["derived"]["rep_bucket_A"], g["derived"]["rep_bucket_B"]],
                                                 dtype=np.float32))
    assert offsets.tolist() == [0, 4, 8] and members.tolist() == list(range(8))
    for qv, top_b, expect_pos, key in [((1.0, 0.0), 1, [0, 1, 2, 3], "attn_dim0_bucket_A_only"),
                                       ((1.0, 0.0), 2, list(range(8)), "attn_dim0_full_read"),
                                       ((0.0, 1.0), 1, [4, 5, 6, 7], "attn_dim0_bucket_B_with_q_0_1")]:
        qq = np.array(qv)
        sel, chosen, _ = O.bucket_select(qq, reps, offsets, members, 7, top_b, 0, 0)
        assert sel.tolist() == expect_pos
        o, _ = O.attention(qq[None, :], K[sel], V[sel], SCALE)
        assert o[0, 0] == pytest.approx(g["derived"][key], rel=1e-13)


def test_lse_merge_of_the_two_buckets(toy):
    g, q, K, V = toy
    a = O.attention(q[None, :], K[:4], V[:4], SCALE)
    b = O.attention(q[None, :], K[4:], V[4:], SCALE)
    o, lse = O.merge_lse([a, b])
    full = O.attention(q[None, :], K, V, SCALE)
    assert o[0, 0] == pytest.approx(g["derived"]["attn_dim0_full_read"], rel=1e-13)
    assert lse[0] == pytest.approx(full[1][0], rel=1e-14)


def test_bucket_step_through_toy(toy):
    """The whole Flat-bucket step (search, expansion, read set, attention) on the eight entries: bucket A alone gives
    the printed 23.24, both buckets the printed 36.45, and q = (0, 1) picks bucket B (63.2422 by hand)."""
    g, q, K, V = toy
    reps, offsets, members = O.bucket_build(K, np.array([0, 0, 0, 0, 1, 1, 1, 1]), 2)
    for qv, top_b, expect_pos, expect_chosen, key in [
            ((1.0, 0.0), 1, [0, 1, 2, 3], [0], "attn_dim0_bucket_A_only"),
            ((1.0, 0.0), 2, list(range(8)), [0, 1], "attn_dim0_full_read"),
            ((0.0, 1.0), 1, [4, 5, 6, 7], [1], "attn_dim0_bucket_B_with_q_0_1")]:
        qq = np.array(qv)
        sel, chosen, o, lse = O.bucket_step(qq, reps, offsets, members, qq[None, :], K, 7, top_b, 0, 0, SCALE, 2,
                                            2, v=V)
        assert sel.tolist() == expect_pos and chosen.tolist() == expect_chosen
        assert o[0, 0] == pytest.approx(g["derived"][key], rel=1e-13)
        assert o[0, 1] == 0.0
        # lse by hand: log of the sum of exp(q.k / sqrt(2)) over the rows read
        assert lse[0] == pytest.approx(math.log(sum(math.exp(SCALE * float(np.dot(qq, K[s]))) for s in expect_pos)),
                                       rel=1e-14)
    # sink and window rows are read on top of the chosen bucket: sink {0} + window {7} + bucket A
    sel, _, o, _ = O.bucket_step(q, reps, offsets, members, q[None, :], K, 7, 1, 1, 1, SCALE, 2, 2, v=V)
    assert sel.tolist() == [1, 2, 3]
    rows = [0, 1, 2, 3, 7]
    z = np.array([SCALE * float(np.dot(q, K[s])) for s in rows])
    e = np.exp(z - z.max())
    assert o[0, 0] == pytest.approx(float(np.dot(e, V[rows, 0]) / e.sum()), rel=1e-13)


def test_dsa_step_through_toy(toy):
    """The whole DSA step with one indexer head (w = 1, q_idx = (1, 0)): top-4 reads bucket A (printed 23.24),
    top-8 reads everything (printed 36.45)."""
    g, q, K, V = toy
    for k, key in [(4, "attn_dim0_bucket_A_only"), (8, "attn_dim0_full_read")]:
        sel, o, lse = O.dsa_step(q[None, :], np.array([1.0]), K, q[None, :], K, 7, k, 0, 0, SCALE, 2, 2, v=V)
        assert sel.tolist() == list(range(k))
        assert o[0, 0] == pytest.approx(g["derived"][key], rel=1e-13)
        assert abs(o[0, 0] - g["printed"][key]) < 0.005
