"""Parity at the full workload sizes, in the launch configuration bench.py times (the same entry points, default
algorithm choices and workspace sizing), checked on sampled queries the oracle can compute one at a time.

Workloads (sa_workloads.configs): 128K decode with 16 queries, the 32768-query prefill chunk, the 1M Flat bucket
search and the 10M decode with e4m3 index keys. Selection follows the band rule of the selection tests; attention
is checked on the read set the GPU selected, at the bf16 tolerance (2e-2 absolute), and the relative error is
reported.
"""
import gc

import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from sa_workloads import gen, get_workload
from tests.gpu_helpers import band_compare, selected, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
ATTN_TOL = 2e-2


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _scores_upto(k_dev, q64, w64, n, chunk=1 << 20):
    """fp32 oracle scores of positions 0..n-1, decoding the stored keys one chunk at a time."""
    out = []
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        kf = to_f64(k_dev[a:b])
        out.append(O.index_score_f32(q64, w64, kf, np.arange(b - a)))
        del kf
    return np.concatenate(out)


def _check_select(inp, wl, b, idx, n_sel):
    t = wl.t_positions()[b]
    q64, w64 = to_f64(inp["q_idx"][b]), inp["w"][b].double().cpu().numpy()
    cand = O.candidate_positions(t, wl.n_sink, wl.n_window)
    sc = _scores_upto(inp["k_idx"], q64, w64, t + 1)[cand]
    ref = O.topk_positions(sc, cand, wl.k_sparse)
    got = selected(idx[b], int(n_sel[b].item()))
    band_compare(got, ref, cand, sc, wl.k_sparse)
    return got


def _check_attn(inp, wl, b, sel, out):
    t = wl.t_positions()[b]
    R = O.read_set(t, wl.n_sink, wl.n_window, sel)
    rows = to_f64(inp["kv"][torch.as_tensor(R, device=inp["kv"].device)])
    ref, _ = O.sparse_attn(to_f64(inp["q"][b]), rows, np.arange(R.size), wl.softmax_scale, wl.d_qk, wl.d_v)
    got = out[b].double().cpu().numpy()
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"query {b}: |R| = {R.size}, max |o - oracle| = {err:.3e}, relative L2 = {rel:.3e}")
    assert err <= ATTN_TOL, (b, err)


def _run_dsa(wl, sample):
    inp = gen.make_inputs(wl, device=DEV)
    t = inp["t"]
    idx, n_sel = sa.sa_select_topk(inp["q_idx"], inp["w"], inp["k_idx"], wl.k_sparse, wl.n_sink, wl.n_window, t=t)
    out = sa.sa_sparse_attn(inp["q"], inp["kv"], idx, n_sel, wl.n_sink, wl.n_window, wl.softmax_scale, t=t,
                            d_v=wl.d_v)
    torch.cuda.synchronize()
    for b in sample:
        sel = _check_select(inp, wl, b, idx, n_sel)
        _check_attn(inp, wl, b, sel, out)
    del inp, idx, n_sel, out
    _free()


def test_dsa_decode_128k_full():
    _run_dsa(get_workload("dsa_decode_128k"), [0, 7, 15])


def test_prefill_chunk_128k_sampled():
    wl = get_workload("prefill_chunk_128k")
    _run_dsa(wl, [0, wl.B // 2 - 1, wl.B - 1])


def test_decode_10m_fp8_full():
    _run_dsa(get_workload("decode_10m_fp8"), [0])


def test_lsa_flat_1m_full():
    wl = get_workload("lsa_flat_1m")
    inp = gen.make_inputs(wl, device=DEV)
    t = inp["t"]
    reps, offsets, members = sa.sa_bucket_build(inp["k_idx"], inp["assign"], wl.n_buckets)
    idx, n_sel, buckets = sa.sa_bucket_select(inp["q_idx"], reps, offsets, members, wl.L, wl.top_b, wl.n_sink,
                                              wl.n_window, cap=8192, t=t, return_buckets=True)
    out = sa.sa_sparse_attn(inp["q"], inp["kv"], idx, n_sel, wl.n_sink, wl.n_window, wl.softmax_scale, t=t,
                            d_v=wl.d_v)
    torch.cuda.synchronize()
    # the directory: CSR bit-exact, representatives within 1e-6 relative
    ref_reps, ref_off, ref_mem = O.bucket_build(to_f64(inp["k_idx"]), inp["assign"].cpu().numpy(), wl.n_buckets)
    np.testing.assert_array_equal(offsets.cpu().numpy(), ref_off)
    np.testing.assert_array_equal(members.cpu().numpy(), ref_mem)
    g = reps.cpu().numpy().astype(np.float64)
    r = ref_reps.astype(np.float64)
    assert np.all(np.abs(g - r) <= 1e-6 * np.maximum(np.abs(r), 1e-30) + 1e-30)
    # selection and attention of sampled queries, with the same representatives on both sides
    reps32 = reps.cpu().numpy()
    off_np, mem_np = offsets.cpu().numpy().astype(np.int64), members.cpu().numpy().astype(np.int64)
    ids = np.nonzero(np.diff(off_np) > 0)[0]
    for b in (0, wl.B - 1):
        tb = wl.t_positions()[b]
        q64 = to_f64(inp["q_idx"][b])
        ref_sel, ref_chosen, sc = O.bucket_select(q64, reps32, off_np, mem_np, tb, wl.top_b, wl.n_sink, wl.n_window)
        ns = int(n_sel[b].item())
        assert ns >= 0, "bucket expansion overflowed its capacity"
        got = selected(idx[b], ns)
        got_chosen = buckets[b].cpu().numpy()
        # bucket level: the band rule on the bucket scores; outside it the chosen buckets agree
        nband = band_compare(np.sort(got_chosen), np.sort(ref_chosen), ids, sc[ids], wl.top_b)
        if nband == 0:
            np.testing.assert_array_equal(got, ref_sel)
        # the expansion of the buckets the GPU chose is exact
        lo = O.sink_positions(tb, wl.n_sink).size
        hi = max(lo, tb - wl.n_window + 1)
        exp = np.concatenate([mem_np[off_np[c]:off_np[c + 1]] for c in got_chosen])
        np.testing.assert_array_equal(got, np.sort(exp[(exp >= lo) & (exp < hi)]))
        _check_attn(inp, wl, b, got, out)
    del inp, reps, offsets, members, idx, n_sel, buckets, out
    _free()
