"""GPU parity of the Tree bucket search (sa_bucket_tree_select) against the oracle (LSA eight-entry page, section 2,
step 3: the Tree variant searches level by level; news page on the open-sourcing of LSA: hierarchical clustering,
cluster centres scanned only).

* Keeping every node reduces the Tree to the Flat search: the GPU result must equal sa_bucket_select's bit for bit
  (the node scores are computed in the same order as the Flat scorer's).
* A hand-built tree whose sums are exact in fp32 (keys on a 1/4 grid, power-of-two buckets, integer queries) must
  match the oracle exactly, ties included.
* Clustered random inputs: the chosen buckets must match the oracle's (run on the GPU-built representatives)
  outside near-ties at the kept-node and top_b boundaries, and the expansion of the GPU's choice must be exact.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from sa_workloads import gen, get_workload
from tests.gpu_helpers import selected, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _build_tree(k, assign, nb, fan):
    """Buckets numbered so that siblings are contiguous: parent of bucket c = c // fan."""
    reps, offsets, members = sa.sa_bucket_build(k, assign, nb)
    n_top = (nb + fan - 1) // fan
    parent = torch.arange(nb, device=DEV, dtype=torch.int32) // fan
    top_reps, _, _ = sa.sa_bucket_build(k, parent[assign.long()], n_top)
    child_off = torch.clamp(torch.arange(n_top + 1, device=DEV, dtype=torch.int32) * fan, max=nb).to(torch.int32)
    return reps, offsets, members, top_reps, child_off


def _oracle_levels(levels):
    return [(lv[0].cpu().numpy(), lv[1].cpu().numpy().astype(np.int64)) for lv in levels]


def test_keep_all_equals_flat_bit_exact():
    wl = get_workload("lsa_flat_1m", L=200_000, n_buckets=4096, B=8)
    inp = gen.make_inputs(wl, device=DEV, seed=11, parts=("index",))
    reps, offsets, members, top_reps, child_off = _build_tree(inp["k_idx"], inp["assign"], 4096, 64)
    ts = [wl.L - 1, 150_000, 99_999, 5000, wl.L - 2, 1000, 70_000, 130_000]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    levels = [(top_reps, child_off, top_reps.shape[0])]
    idx, nsel, bk = sa.sa_bucket_tree_select(inp["q_idx"], levels, reps, offsets, members, wl.L, 32, 4, 128, t=t,
                                             return_buckets=True)
    fidx, fnsel, fbk = sa.sa_bucket_select(inp["q_idx"], reps, offsets, members, wl.L, 32, 4, 128, t=t,
                                           return_buckets=True)
    torch.cuda.synchronize()
    assert torch.equal(bk, fbk) and torch.equal(nsel, fnsel) and torch.equal(idx, fidx)


def test_hand_built_exact_with_ties():
    # 256 positions, 32 buckets of 8 (bucket c = positions 8c .. 8c + 7), 8 parents of 4 buckets; keys on a 1/4 grid
    # so every mean and every dot product with an integer query is exact; many equal scores
    g = torch.Generator(device="cpu").manual_seed(3)
    d = 16
    k = (torch.randint(-4, 5, (256, d), generator=g).float() / 4).to(DEV)
    assign = (torch.arange(256) // 8).to(torch.int32).to(DEV)
    reps, offsets, members, top_reps, child_off = _build_tree(k, assign, 32, 4)
    q = torch.randint(-1, 2, (6, d), generator=g).float().to(DEV)
    ts = [255, 200, 130, 63, 17, 5]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    for keep, top_b in [(1, 2), (3, 5), (8, 9)]:
        levels = [(top_reps, child_off, keep)]
        idx, nsel, bk = sa.sa_bucket_tree_select(q, levels, reps, offsets, members, 256, top_b, 2, 6, t=t, cap=256,
                                                 return_buckets=True)
        torch.cuda.synchronize()
        lv = _oracle_levels(levels)
        r32, off, mem = reps.cpu().numpy(), offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
        for b in range(6):
            pos, chosen, _ = O.tree_select(to_f64(q[b]), lv, r32, off, mem, ts[b], [keep], top_b, 2, 6)
            got = bk[b].cpu().numpy()
            np.testing.assert_array_equal(got[got >= 0], chosen)
            np.testing.assert_array_equal(selected(idx[b], int(nsel[b].item())), pos)


def _near_tie(s32, ids, k, rel=1e-5):
    """True if the k-th best of s32[ids] (desc) has another score within rel of it."""
    if ids.size <= k:
        return False
    s = np.sort(s32[ids].astype(np.float64))[::-1]
    kth = s[k - 1]
    return np.sum(np.abs(s - kth) <= rel * max(abs(kth), 1e-30)) > 1


@pytest.mark.parametrize("depth", [2, 3])
def test_clustered_matches_oracle(depth):
    wl = get_workload("lsa_flat_1m", L=300_000, n_buckets=4096, B=8)
    inp = gen.make_inputs(wl, device=DEV, seed=12, parts=("index",))
    reps, offsets, members, mid_reps, mid_off = _build_tree(inp["k_idx"], inp["assign"], 4096, 32)   # 128 mid
    if depth == 2:
        levels = [(mid_reps, mid_off, 16)]
    else:
        # a root level over the 128 mid nodes, 16 per root: root of bucket c = (c // 32) // 16
        root_of_bucket = (torch.arange(4096, device=DEV, dtype=torch.int32) // 32) // 16
        root_reps, _, _ = sa.sa_bucket_build(inp["k_idx"], root_of_bucket[inp["assign"].long()], 8)
        root_off = (torch.arange(9, device=DEV, dtype=torch.int32) * 16).to(torch.int32)
        levels = [(root_reps, root_off, 4), (mid_reps, mid_off, 12)]
    ts = [wl.L - 1, 250_000, 123_456, 20_000, wl.L - 7, 3000, 200_001, 88_888]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel, bk = sa.sa_bucket_tree_select(inp["q_idx"], levels, reps, offsets, members, wl.L, 32, 4, 128, t=t,
                                             return_buckets=True)
    torch.cuda.synchronize()
    lv = _oracle_levels(levels)
    keeps = [x[2] for x in levels]
    r32, off, mem = reps.cpu().numpy(), offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    qf = to_f64(inp["q_idx"])
    exact = 0
    for b in range(wl.B):
        pos, chosen, kept = O.tree_select(qf[b], lv, r32, off, mem, ts[b], keeps, 32, 4, 128)
        got = bk[b].cpu().numpy()
        got = got[got >= 0]
        # near-ties at any kept-node boundary or at the top_b boundary may legitimately flip the choice
        ties = False
        cand = np.arange(lv[0][0].shape[0])
        for (rl, co), keep, kp in zip(lv, keeps, kept):
            s = O.bucket_scores_f32(qf[b], rl)
            ids = cand[np.diff(co)[cand] > 0]
            ties |= _near_tie(s, ids, keep)
            cand = np.concatenate([np.arange(co[c], co[c + 1]) for c in kp])
        s = O.bucket_scores_f32(qf[b], r32)
        ties |= _near_tie(s, cand[np.diff(off)[cand] > 0], 32)
        if not ties:
            np.testing.assert_array_equal(got, chosen)
            exact += 1
        # the expansion of whatever buckets the GPU chose is exact
        exp_pos = np.concatenate([mem[off[c]:off[c + 1]] for c in got]) if got.size else np.zeros(0, np.int64)
        lo, hi = O.sink_positions(ts[b], 4).size, max(O.sink_positions(ts[b], 4).size, ts[b] - 128 + 1)
        np.testing.assert_array_equal(selected(idx[b], int(nsel[b].item())),
                                      np.sort(exp_pos[(exp_pos >= lo) & (exp_pos < hi)]))
    assert exact >= wl.B // 2
