"""GPU parity of the coarse-to-fine index (sa_hi_build, sa_hi_select) against the oracle (LongCat deep-dive,
section "Mechanism 3: hierarchical indexing (HI)"; indexer equation of the DSA baseline section; sink/window budget
of the SI section).

* The mean keys are compared bit for bit (fp64 sums of bf16 keys are exact; both sides round fp64 -> fp32 -> bf16).
* Integer-valued q, k, w make the means multiples of 1/sub_block, and every page and token score exact: the recalled
  pages and the selected positions must match bit for bit, ties included.
* Normal inputs: the recalled pages agree outside the band of pages whose score lies near the M-th page score; the
  token stage is then checked exactly against the oracle's selection over the GPU's own recalled pages (band
  comparison at the k-th token score, as for the flat selection).
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from tests.gpu_helpers import band_compare, selected, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(seed, B, H, d, L, integer, k_pad=0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    if integer:
        q = torch.randint(-2, 3, (B, H, d), generator=g).float()
        k = torch.randint(-2, 3, (L, d + k_pad), generator=g).float()
        w = torch.randint(0, 3, (B, H), generator=g).float()
    else:
        q = torch.randn((B, H, d), generator=g)
        k = torch.randn((L, d + k_pad), generator=g)
        w = torch.randn((B, H), generator=g)
    kk = k.to(torch.bfloat16).to(DEV)
    return q.to(torch.bfloat16).to(DEV), w.to(DEV), kk[:, :d]


def _pages(row: torch.Tensor) -> np.ndarray:
    r = row.cpu().numpy().astype(np.int64)
    n = int(np.sum(r >= 0))
    assert np.all(r[n:] == -1), "page padding must be -1"
    assert np.all(np.diff(r[:n]) > 0), "recalled pages must be strictly ascending"
    return r[:n]


@pytest.mark.parametrize("L,sub,pad", [(10003, 8, 0), (4096, 16, 64), (777, 64, 0), (1, 8, 0)])
def test_means_bit_exact(L, sub, pad):
    _, _, k = _inputs(1, 1, 1, 128, L, integer=False, k_pad=pad)
    k = k * 3.0 if pad == 0 else k     # a wider spread of exponents (still exact in fp64)
    means = sa.sa_hi_build(k, sub)
    torch.cuda.synchronize()
    ref = O.hi_means(to_f64(k), sub)
    np.testing.assert_array_equal(to_f64(means), ref)


def _check_exact(q, w, k, t, sub, P, M, kk, n_sink, n_window):
    B = q.shape[0]
    L = k.shape[0]
    means = sa.sa_hi_build(k, sub)
    tt = None if t is None else torch.tensor(t, dtype=torch.int32, device=DEV)
    idx, n_sel, pages = sa.sa_hi_select(q, w, k, means, sub, P, M, kk, n_sink, n_window, t=tt, return_pages=True)
    torch.cuda.synchronize()
    qf, wf, kf, mf = to_f64(q), w.double().cpu().numpy(), to_f64(k), to_f64(means)
    for b in range(B):
        tb = L - 1 if t is None else t[b]
        ref, ref_pages, _, _, _ = O.hi_select(qf[b], wf[b], kf, mf, tb, P, sub, M, kk, n_sink, n_window)
        np.testing.assert_array_equal(_pages(pages[b]), ref_pages)
        np.testing.assert_array_equal(selected(idx[b], int(n_sel[b].item())), ref)


@pytest.mark.parametrize("H", [64, 32])
@pytest.mark.parametrize("B", [6, 9])
def test_integer_exact_with_ties(H, B):
    L = 40000
    q, w, k = _inputs(5, B, H, 128, L, integer=True)
    ts = [L - 1, 39000, 20000, 17000, 5000, 900, 33333, 123, 39999][:B]
    _check_exact(q, w, k, ts, sub=8, P=128, M=64, kk=700, n_sink=3, n_window=50)


@pytest.mark.parametrize("sub,P", [(64, 64), (4, 256), (2, 128), (16, 1024)])
def test_integer_exact_page_shapes(sub, P):
    # one sub-block per page up to 64 per page; a short cache with a partial last page and last sub-block
    L = 23_457
    q, w, k = _inputs(7, 5, 64, 128, L, integer=True)
    _check_exact(q, w, k, [L - 1, 20000, 4000, 640, 3], sub=sub, P=P, M=12, kk=300, n_sink=4, n_window=128)


def test_integer_exact_budget_larger_than_pages():
    # k larger than every candidate in the recalled pages: all of them, sink and window excluded
    L = 30000
    q, w, k = _inputs(8, 4, 64, 128, L, integer=True)
    _check_exact(q, w, k, [L - 1, 15000, 700, 200], sub=8, P=128, M=8, kk=2048, n_sink=4, n_window=128)


def test_integer_exact_decode_no_t_padded_keys():
    L = 50000
    q, w, k = _inputs(9, 3, 64, 128, L, integer=True, k_pad=64)   # k_ld = 192 elements
    _check_exact(q, w, k, None, sub=8, P=128, M=100, kk=1000, n_sink=0, n_window=0)


def test_all_pages_recalled_equals_flat_selection():
    """M at least the number of pages: the token stage sees every candidate, so the result is the flat top-k."""
    L, B, kk = 20000, 5, 1500
    q, w, k = _inputs(10, B, 64, 128, L, integer=False)
    ts = [L - 1, 12345, 5000, 600, 64]
    tt = torch.tensor(ts, dtype=torch.int32, device=DEV)
    means = sa.sa_hi_build(k, 8)
    idx, n_sel = sa.sa_hi_select(q, w, k, means, 8, 128, 1024, kk, 4, 128, t=tt)
    flat_idx, flat_n = sa.sa_select_topk(q, w, k, kk, 4, 128, t=tt)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 4, 128)
        got = selected(idx[b], int(n_sel[b].item()))
        band_compare(got, ref, cand, sc, kk)
        np.testing.assert_array_equal(got, selected(flat_idx[b], int(flat_n[b].item())))


def _check_normal(q, w, k, t, sub, P, M, kk, n_sink, n_window, stride=1):
    """Pages outside the score band must match the oracle's; the token stage is exact given the recalled pages.
    Queries b = 0, stride, 2 stride, ... are checked (the oracle's token scores are the slow part)."""
    B = q.shape[0]
    L = k.shape[0]
    means = sa.sa_hi_build(k, sub)
    tt = None if t is None else torch.tensor(t, dtype=torch.int32, device=DEV)
    idx, n_sel, pages = sa.sa_hi_select(q, w, k, means, sub, P, M, kk, n_sink, n_window, t=tt, return_pages=True)
    torch.cuda.synchronize()
    qf, wf, kf, mf = to_f64(q), w.double().cpu().numpy(), to_f64(k), to_f64(means)
    np.testing.assert_array_equal(to_f64(means), O.hi_means(kf, sub))
    for b in range(0, B, stride):
        tb = L - 1 if t is None else t[b]
        psc, pids = O.hi_page_scores(qf[b], wf[b], mf, P // sub, tb, P)
        ref_pages = O.topk_positions(psc, pids, M)
        got_pages = _pages(pages[b])
        assert got_pages.size == ref_pages.size
        assert np.all(got_pages <= tb // P)
        if ref_pages.size < pids.size:
            # the page band: scores within 1e-4 of the largest page-score magnitude from the M-th page score
            mth = np.sort(psc.astype(np.float64))[::-1][M - 1]
            band = pids[np.abs(psc.astype(np.float64) - mth) <= 1e-4 * np.abs(psc).max()]
            np.testing.assert_array_equal(np.setdiff1d(got_pages, band), np.setdiff1d(ref_pages, band))
        cand = O.candidate_positions(tb, n_sink, n_window)
        cand = cand[np.isin(cand // P, got_pages)]
        sc = O.index_score_f32(qf[b], wf[b], kf, cand)
        ref = O.topk_positions(sc, cand, kk)
        band_compare(selected(idx[b], int(n_sel[b].item())), ref, cand, sc, kk)


@pytest.mark.parametrize("H", [64, 32])
def test_normal_inputs_decode(H):
    L = 100_000
    q, w, k = _inputs(11, 5, H, 128, L, integer=False)
    _check_normal(q, w, k, [L - 1, 99_000, 50_000, 7000, 130], sub=8, P=128, M=32, kk=2048, n_sink=4, n_window=128)


def test_normal_inputs_prefill_chunk():
    """A causal prefill chunk: 64 consecutive queries at the end of a 64K cache, recalled pages per query."""
    L, B = 65536, 64
    q, w, k = _inputs(12, B, 64, 128, L, integer=False)
    ts = list(range(L - B, L))
    _check_normal(q, w, k, ts, sub=8, P=128, M=64, kk=2048, n_sink=4, n_window=128, stride=9)


def test_max_recalled_pages_and_union():
    """M = 1024 pages per query over a cache of 4096 pages; four queries per workgroup walk a union of up to 4096
    pages (the limits of the token stage's LDS lists)."""
    L, B = 4096 * 128, 4
    q, w, k = _inputs(13, B, 64, 128, L, integer=False)
    _check_normal(q, w, k, None, sub=8, P=128, M=1024, kk=2048, n_sink=4, n_window=128, stride=3)
