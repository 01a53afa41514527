"""GPU parity of sa_bucket_build and sa_bucket_select against the oracle (LSA eight-entry page, section 2: buckets
keep a representative and their member positions; Flat search over representatives; chosen buckets expand to
positions, plus sink and window)."""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from sa_workloads import gen, get_workload
from tests.gpu_helpers import band_compare, selected, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _small_lsa(seed, L=60000, nb=1000, B=4):
    wl = get_workload("lsa_flat_1m", L=L, n_buckets=nb, B=B)
    inp = gen.make_inputs(wl, device=DEV, seed=seed, parts=("index",))
    return wl, inp


@pytest.mark.parametrize("seed", [0, 1])
def test_build_matches_oracle(seed):
    wl, inp = _small_lsa(seed)
    reps, offsets, members = sa.sa_bucket_build(inp["k_idx"], inp["assign"], wl.n_buckets)
    torch.cuda.synchronize()
    r_o, off_o, mem_o = O.bucket_build(to_f64(inp["k_idx"]), inp["assign"].cpu().numpy(), wl.n_buckets)
    np.testing.assert_array_equal(offsets.cpu().numpy(), off_o)
    np.testing.assert_array_equal(members.cpu().numpy(), mem_o)
    # fp64 sums rounded once: equal up to the summation order (at most one fp32 ulp)
    np.testing.assert_allclose(reps.cpu().numpy(), r_o, rtol=2 ** -23, atol=1e-30)


def test_build_toy_and_empty_buckets():
    K = [[1, 0], [0.8, 0.2], [0.6, 0.4], [0.4, 0.6], [0, 1], [-0.2, 0.8], [-0.4, 0.6], [-0.6, 0.4]]
    k = torch.zeros((8, 4), dtype=torch.float32, device=DEV)   # rows padded to 16 bytes
    k[:, :2] = torch.tensor(K, device=DEV)
    assign = torch.tensor([0, 0, 0, 0, 2, 2, 2, 2], dtype=torch.int32, device=DEV)
    reps, offsets, members = sa.sa_bucket_build(k, assign, 3)
    assert offsets.tolist() == [0, 4, 4, 8] and members.tolist() == list(range(8))
    r = reps.cpu().numpy()
    np.testing.assert_allclose(r[0, :2], [0.7, 0.3], rtol=1e-7)
    np.testing.assert_allclose(r[2, :2], [-0.3, 0.7], rtol=1e-7)
    assert np.all(r[1] == 0)


@pytest.mark.parametrize("seed", [0, 1])
def test_select_matches_oracle(seed):
    wl, inp = _small_lsa(seed)
    L, B = wl.L, wl.B
    reps, offsets, members = sa.sa_bucket_build(inp["k_idx"], inp["assign"], wl.n_buckets)
    ts = [L - 1, L - 5000, 30000, 100]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel, buckets = sa.sa_bucket_select(inp["q_idx"], reps, offsets, members, L, 32, 4, 128, cap=8192, t=t,
                                             return_buckets=True)
    torch.cuda.synchronize()
    qf = to_f64(inp["q_idx"])
    r32, off, mem = reps.cpu().numpy(), offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    for b in range(B):
        ref_pos, ref_chosen, sc = O.bucket_select(qf[b], r32, off, mem, ts[b], 32, 4, 128)
        ids = np.nonzero(np.diff(off) > 0)[0]
        got_chosen = buckets[b].cpu().numpy()
        nband = band_compare(np.sort(got_chosen), np.sort(ref_chosen), ids, sc[ids], 32)
        if nband == 0:
            np.testing.assert_array_equal(got_chosen, ref_chosen)     # order: score desc, id asc
            np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref_pos)
        # the expansion of whatever buckets the GPU chose must be exact
        exp_pos = np.concatenate([mem[off[c]:off[c + 1]] for c in got_chosen])
        lo, hi = O.sink_positions(ts[b], 4).size, max(O.sink_positions(ts[b], 4).size, ts[b] - 128 + 1)
        exp_pos = np.sort(exp_pos[(exp_pos >= lo) & (exp_pos < hi)])
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), exp_pos)


def test_select_overflow_reports_needed():
    wl, inp = _small_lsa(3)
    reps, offsets, members = sa.sa_bucket_build(inp["k_idx"], inp["assign"], wl.n_buckets)
    idx, nsel = sa.sa_bucket_select(inp["q_idx"], reps, offsets, members, wl.L, 32, 4, 128, cap=16)
    torch.cuda.synchronize()
    assert torch.all(nsel < -16) and torch.all(idx == -1)


def test_singleton_buckets_reduce_to_plain_topk():
    """One position per bucket: rep = key and the search is a plain top-k of q.k."""
    L, d, B, top = 3000, 16, 2, 40
    g = torch.Generator(device="cpu").manual_seed(4)
    k = torch.randint(-2, 3, (L, d), generator=g).float().to(DEV)
    q = torch.randint(-2, 3, (B, d), generator=g).float().to(DEV)
    assign = torch.arange(L, dtype=torch.int32, device=DEV)
    reps, offsets, members = sa.sa_bucket_build(k, assign, L)
    idx, nsel = sa.sa_bucket_select(q, reps, offsets, members, L, top, 0, 0, cap=64)
    torch.cuda.synchronize()
    kf, qf = k.double().cpu().numpy(), q.double().cpu().numpy()
    for b in range(B):
        sc = (kf @ qf[b]).astype(np.float32)
        ref = O.topk_positions(sc, np.arange(L), top)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)


@pytest.mark.parametrize("layout", ["contiguous", "large"])
def test_expand_clustered_and_large(layout):
    """Expansions whose positions crowd a few of the sort's position bins: buckets of contiguous positions, and a
    few very large buckets (about 12K positions per query). The expansion must still be the exact ascending union."""
    if layout == "contiguous":
        L, d, B, nb, top, cap = 200000, 16, 3, 3125, 24, 4096     # bucket c = positions 64c .. 64c + 63
        assign_np = (np.arange(L) // 64).astype(np.int32)
    else:
        L, d, B, nb, top, cap = 200000, 16, 3, 64, 4, 16384       # about 3125 positions per bucket
        assign_np = np.random.default_rng(5).integers(0, nb, L).astype(np.int32)
    g = torch.Generator(device="cpu").manual_seed(6)
    k = torch.randn((L, d), generator=g).to(DEV)
    q = torch.randn((B, d), generator=g).to(DEV)
    assign = torch.as_tensor(assign_np, device=DEV)
    reps, offsets, members = sa.sa_bucket_build(k, assign, nb)
    ts = [L - 1, L // 2, 150000]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel, buckets = sa.sa_bucket_select(q, reps, offsets, members, L, top, 4, 64, cap=cap, t=t,
                                             return_buckets=True)
    torch.cuda.synchronize()
    off, mem = offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    for b in range(B):
        chosen = buckets[b].cpu().numpy()
        exp_pos = np.concatenate([mem[off[c]:off[c + 1]] for c in chosen])
        lo, hi = 4, ts[b] - 64 + 1
        exp_pos = np.sort(exp_pos[(exp_pos >= lo) & (exp_pos < hi)])
        assert exp_pos.size > (500 if layout == "contiguous" else 3000)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), exp_pos)


def test_choice_ties_long_rows_and_few_nonempty():
    """Integer keys: every score is exact and ties are heavy. 20000 buckets of two members each (a row longer than
    the part of the choice held in registers): the chosen ids, in rank order (score desc, id asc), and the
    expanded positions match the oracle exactly. Then only 10 of 40 buckets hold members and top_b = 16: every
    non-empty bucket is chosen and -1 pads the rank list."""
    g = torch.Generator(device="cpu").manual_seed(6)
    L, d, B, nb, top = 40000, 16, 3, 20000, 50
    k = torch.randint(-2, 3, (L, d), generator=g).float().to(DEV)
    q = torch.randint(-2, 3, (B, d), generator=g).float().to(DEV)
    assign = (torch.arange(L) % nb).to(torch.int32).to(DEV)
    reps, offsets, members = sa.sa_bucket_build(k, assign, nb)
    idx, nsel, buckets = sa.sa_bucket_select(q, reps, offsets, members, L, top, 0, 0, cap=200, return_buckets=True)
    torch.cuda.synchronize()
    qf = q.double().cpu().numpy()
    r32, off, mem = reps.cpu().numpy(), offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    for b in range(B):
        ref_pos, ref_chosen, sc = O.bucket_select(qf[b], r32, off, mem, L - 1, top, 0, 0)
        assert np.unique(sc).size < nb / 10                           # ties are really exercised
        np.testing.assert_array_equal(buckets[b].cpu().numpy(), ref_chosen)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref_pos)

    L2, nb2, top2 = 500, 40, 16
    k2 = torch.randint(-2, 3, (L2, d), generator=g).float().to(DEV)
    assign2 = ((torch.arange(L2) % 10) * 4).to(torch.int32).to(DEV)     # buckets 0, 4, ..., 36
    reps2, off2, mem2 = sa.sa_bucket_build(k2, assign2, nb2)
    idx2, nsel2, buckets2 = sa.sa_bucket_select(q, reps2, off2, mem2, L2, top2, 0, 0, cap=512, return_buckets=True)
    torch.cuda.synchronize()
    o2, m2 = off2.cpu().numpy().astype(np.int64), mem2.cpu().numpy().astype(np.int64)
    for b in range(B):
        ref_pos, ref_chosen, sc = O.bucket_select(qf[b], reps2.cpu().numpy(), o2, m2, L2 - 1, top2, 0, 0)
        assert ref_chosen.size == 10
        got = buckets2[b].cpu().numpy()
        np.testing.assert_array_equal(got[:10], ref_chosen)
        assert np.all(got[10:] == -1)
        np.testing.assert_array_equal(selected(idx2[b], nsel2[b].item()), np.arange(L2))


@pytest.mark.parametrize("n_mid", [100, 1000])
def test_choice_first_bin_candidates(n_mid):
    """Singleton buckets with exact scores: 20 at 6.0, n_mid at 4.25 / 4.5 / 4.75 (heavy ties), the rest at 1.0.
    With top_b = 32 the 32nd score lies in the bin [4, 5) of the first digit pass, which then holds 20 + n_mid
    candidates: few enough to be ranked directly (100), or too many (1000), so that the remaining digit passes and
    the tie limit decide. Either way the chosen ids, in rank order (score desc, id asc), match the oracle."""
    L, d, nb, top = 3000, 4, 3000, 32
    rng = np.random.default_rng(7 + n_mid)
    vals = np.full(L, 1.0)
    ids = rng.permutation(L)
    vals[ids[:20]] = 6.0
    vals[ids[20:20 + n_mid]] = rng.choice([4.25, 4.5, 4.75], n_mid)
    k_np = np.zeros((L, d), dtype=np.float32)
    k_np[:, 0] = vals
    k = torch.as_tensor(k_np, device=DEV)
    q = torch.tensor([[1.0, 0, 0, 0], [2.0, 0, 0, 0]], device=DEV)
    assign = torch.arange(L, dtype=torch.int32, device=DEV)
    reps, offsets, members = sa.sa_bucket_build(k, assign, nb)
    idx, nsel, buckets = sa.sa_bucket_select(q, reps, offsets, members, L, top, 0, 0, cap=64, return_buckets=True)
    torch.cuda.synchronize()
    qf = q.double().cpu().numpy()
    r32, off, mem = reps.cpu().numpy(), offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    for b in range(2):
        ref_pos, ref_chosen, sc = O.bucket_select(qf[b], r32, off, mem, L - 1, top, 0, 0)
        np.testing.assert_array_equal(buckets[b].cpu().numpy(), ref_chosen)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref_pos)


def test_select_prefilled_workspace():
    """The bucket search gives the same result whatever its workspace held before (all-ones bytes, a byte pattern,
    zeros): every slot key it reads is written by the same call."""
    wl, inp = _small_lsa(2)
    reps, offsets, members = sa.sa_bucket_build(inp["k_idx"], inp["assign"], wl.n_buckets)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=DEV)
    res = []
    for fill in (0xFF, 0x5A, 0x00):
        ws.fill_(fill)
        idx, nsel, buckets = sa.sa_bucket_select(inp["q_idx"], reps, offsets, members, wl.L, 32, 4, 128, cap=8192,
                                                 return_buckets=True, ws=ws)
        torch.cuda.synchronize()
        res.append((idx.cpu(), nsel.cpu(), buckets.cpu()))
    for r in res[1:]:
        for a, b in zip(res[0], r):
            assert torch.equal(a, b)
    qf = to_f64(inp["q_idx"])
    r32, off, mem = reps.cpu().numpy(), offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    ids = np.nonzero(np.diff(off) > 0)[0]
    for b in range(wl.B):
        ref_pos, ref_chosen, sc = O.bucket_select(qf[b], r32, off, mem, wl.L - 1, 32, 4, 128)
        nband = band_compare(np.sort(res[0][2][b].numpy()), np.sort(ref_chosen), ids, sc[ids], 32)
        if nband == 0:
            np.testing.assert_array_equal(res[0][2][b].numpy(), ref_chosen)
            np.testing.assert_array_equal(selected(res[0][0][b], res[0][1][b].item()), ref_pos)
