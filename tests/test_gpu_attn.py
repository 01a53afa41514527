"""GPU parity of sa_sparse_attn against the oracle (LongCat deep-dive, DSA baseline section, sparse-attention
equation; SI section, sink/window rows and the LSE merge). fp32 within 1e-5 abs, bf16 within 2e-2 abs."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from sa_workloads import gen, get_workload
from tests.gpu_helpers import to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rand_sparse(rng, t, n_sink, n_window, n):
    cand = O.candidate_positions(t, n_sink, n_window)
    n = min(n, cand.size)
    return np.sort(rng.choice(cand, size=n, replace=False)) if n else np.zeros(0, np.int64)


def _pack_idx(sel_list, idx_ld):
    B = len(sel_list)
    idx = np.full((B, idx_ld), -1, np.int32)
    nsel = np.zeros(B, np.int32)
    for b, s in enumerate(sel_list):
        idx[b, :len(s)] = s
        nsel[b] = len(s)
    return torch.tensor(idx, device=DEV), torch.tensor(nsel, device=DEV)


def test_toy_eight_entries_fp32():
    """The LSA eight-entry example: q=(1,0), scale 1/sqrt(2); full read 36.4517, bucket A only 23.2422."""
    K = [[1, 0], [0.8, 0.2], [0.6, 0.4], [0.4, 0.6], [0, 1], [-0.2, 0.8], [-0.4, 0.6], [-0.6, 0.4]]
    V = [[10 * (i + 1), 0] for i in range(8)]
    kv = torch.tensor(K, dtype=torch.float32, device=DEV)
    v = torch.tensor(V, dtype=torch.float32, device=DEV)
    q = torch.tensor([[[1.0, 0.0]]], device=DEV)
    for sel, expect in [(list(range(8)), 36.4517124248522), ([0, 1, 2, 3], 23.2421743979185)]:
        idx, nsel = _pack_idx([np.array(sel)], 8)
        o = sa.sa_sparse_attn(q, kv, idx, nsel, 0, 0, 1 / math.sqrt(2), v=v)
        torch.cuda.synchronize()
        assert abs(o[0, 0, 0].item() - expect) < 1e-5 and o[0, 0, 1].item() == 0.0
    # the same rows as sink + window: t=7, sink 4, window 4, no sparse part
    o = sa.sa_sparse_attn(q, kv, None, None, 4, 4, 1 / math.sqrt(2), v=v)
    assert abs(o[0, 0, 0].item() - 36.4517124248522) < 1e-5


@pytest.mark.parametrize("seed", [0, 1])
def test_toy_decode_config_fp32(seed):
    """1 query, 1 head, width 64 used as K and V, sink 4 + window 32 + 64 sparse rows, scale 1/8 (generic path)."""
    wl = get_workload("toy_decode_f32")
    inp = gen.make_inputs(wl, device=DEV, seed=seed, parts=("attn",))
    rng = np.random.default_rng(seed)
    t = wl.L - 1
    sel = _rand_sparse(rng, t, wl.n_sink, wl.n_window, wl.k_sparse)
    idx, nsel = _pack_idx([sel], wl.k_sparse)
    o, lse = sa.sa_sparse_attn(inp["q"], inp["kv"], idx, nsel, wl.n_sink, wl.n_window, wl.softmax_scale,
                               return_lse=True)
    R = O.read_set(t, wl.n_sink, wl.n_window, sel)
    assert R.size == 100
    oo, ol = O.sparse_attn(to_f64(inp["q"][0]), to_f64(inp["kv"]), R, wl.softmax_scale, 64, 64)
    np.testing.assert_allclose(o[0].double().cpu().numpy(), oo, atol=1e-5, rtol=0)
    np.testing.assert_allclose(lse[0].double().cpu().numpy(), ol, atol=1e-5, rtol=0)


def _mfma_case(seed, B, L, n_list, n_sink, n_window, d_v, q_scale=1.0, t=None, H=128, idx_ld=None, ws_fill=None,
               scale=None):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = (torch.randn((B, H, 576), generator=g) * q_scale).to(torch.bfloat16).to(DEV)
    kv = torch.randn((L, 576), generator=g).to(torch.bfloat16).to(DEV)
    rng = np.random.default_rng(seed)
    ts = [L - 1] * B if t is None else t
    sels = [_rand_sparse(rng, ts[b], n_sink, n_window, n_list[b]) for b in range(B)]
    idx_ld = max(1, max(n_list)) if idx_ld is None else idx_ld
    idx, nsel = _pack_idx(sels, idx_ld)
    tt = torch.tensor(ts, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(576) if scale is None else scale
    ws = None
    if ws_fill is not None:  # every workspace byte set, e.g. 0xFF: NaN in every float no kernel writes
        nb = sa.sa_sparse_attn_workspace(B, H, 576, d_v, n_sink + n_window + idx_ld, sa.SA_BF16)
        ws = torch.full((max(nb, 1),), ws_fill, dtype=torch.uint8, device=DEV)
    o, lse = sa.sa_sparse_attn(q, kv, idx, nsel, n_sink, n_window, scale, t=tt, d_v=d_v, return_lse=True, ws=ws)
    torch.cuda.synchronize()
    qf, kvf = to_f64(q), to_f64(kv)
    worst = 0.0
    for b in range(B):
        R = O.read_set(ts[b], n_sink, n_window, sels[b])
        oo, ol = O.sparse_attn(qf[b], kvf, R, scale, 576, d_v)
        got = o[b].double().cpu().numpy()
        err = np.abs(got - oo).max()
        worst = max(worst, err)
        assert err < 2e-2, (b, err)
        np.testing.assert_allclose(lse[b].double().cpu().numpy(), ol, atol=2e-3, rtol=0)
    return worst


@pytest.mark.parametrize("d_v", [576, 512])
def test_mfma_ragged_and_splits(d_v):
    # ragged read sets (not multiples of 32), one empty sparse part, one that needs several splits
    _mfma_case(0, B=4, L=8192, n_list=[2048, 77, 0, 1500], n_sink=4, n_window=128, d_v=d_v)


def test_mfma_read_sets_far_below_bound():
    # the grid is planned for idx_ld + sink + window rows; the actual read sets are far smaller, end on and off
    # tile boundaries, and leave most splits of a query empty
    # (splits with no rows leave their workspace rows unwritten: a NaN-filled workspace must not reach the output)
    _mfma_case(5, B=5, L=20000, n_list=[100, 1000, 0, 32 * 40 - 132, 6000], n_sink=4, n_window=128, d_v=576,
               idx_ld=8192, ws_fill=0xFF)


@pytest.mark.parametrize("H", [64, 192])
def test_mfma_head_groups(H):
    # one and three 64-head groups per query (the block mapping interleaves a unit's head groups): ragged read sets,
    # several splits per query
    _mfma_case(6, B=3, L=9000, n_list=[1500, 33, 700], n_sink=4, n_window=128, d_v=576, H=H)


def test_mfma_single_split_and_peaked():
    # many queries -> one split each; queries x8 give peaked softmax with |o| ~ |V|
    _mfma_case(1, B=64, L=4096, n_list=[40] * 64, n_sink=0, n_window=0, d_v=576, q_scale=8.0)


def test_mfma_short_prefix_t():
    # per-query t: sink and window overlap the whole visible prefix for early queries
    _mfma_case(2, B=3, L=5000, n_list=[0, 10, 300], n_sink=4, n_window=128, d_v=576, t=[2, 200, 4999])


@pytest.mark.parametrize("scale", [0.0, -1 / math.sqrt(576), -0.2])
def test_mfma_zero_and_negative_scale(scale):
    # any finite scale is valid: a zero scale averages V over the read set (lse = ln |R|), a negative one prefers
    # the rows least aligned with q; ragged read sets put masked rows in the last tile of each split
    _mfma_case(7, B=3, L=6000, n_list=[1000, 45, 333], n_sink=4, n_window=128, d_v=576, scale=scale)


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_generic_zero_and_negative_scale(scale):
    B, H, d, L = 2, 3, 64, 500
    g = torch.Generator(device="cpu").manual_seed(8)
    q = torch.randn((B, H, d), generator=g).to(DEV)
    kv = torch.randn((L, d), generator=g).to(DEV)
    rng = np.random.default_rng(8)
    sels = [_rand_sparse(rng, L - 1, 2, 10, n) for n in (50, 7)]
    idx, nsel = _pack_idx(sels, 50)
    o, lse = sa.sa_sparse_attn(q, kv, idx, nsel, 2, 10, scale, return_lse=True)
    torch.cuda.synchronize()
    for b in range(B):
        R = O.read_set(L - 1, 2, 10, sels[b])
        oo, ol = O.sparse_attn(to_f64(q[b]), to_f64(kv), R, scale, d, d)
        np.testing.assert_allclose(o[b].double().cpu().numpy(), oo, atol=1e-5, rtol=0)
        np.testing.assert_allclose(lse[b].double().cpu().numpy(), ol, atol=1e-5, rtol=0)


def test_mfma_empty_read_set():
    q = torch.randn((2, 128, 576), device=DEV).to(torch.bfloat16)
    kv = torch.randn((100, 576), device=DEV).to(torch.bfloat16)
    idx = torch.full((2, 8), -1, dtype=torch.int32, device=DEV)
    nsel = torch.zeros(2, dtype=torch.int32, device=DEV)
    o, lse = sa.sa_sparse_attn(q, kv, idx, nsel, 0, 0, 0.1, return_lse=True)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_dense_reduction_bf16():
    """k >= |C|: reading every visible row equals dense softmax attention (oracle, fp64)."""
    L = 700
    _mfma_case(3, B=2, L=L, n_list=[L - 4 - 64] * 2, n_sink=4, n_window=64, d_v=576)


@pytest.mark.parametrize("dtype,tol", [("bf16", 2e-2), ("f32", 1e-5)])
def test_generic_separate_v(dtype, tol):
    """A separate V cache (wider than K), several queries and heads, ragged read sets with t given: the generic
    kernel against the oracle, and the lse within its own tolerance."""
    B, H, d_qk, d_v, L = 4, 6, 64, 96, 3000
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(21)
    q = torch.randn((B, H, d_qk), generator=g).to(dt).to(DEV)
    kv = torch.randn((L, d_qk), generator=g).to(dt).to(DEV)
    v = torch.randn((L, d_v), generator=g).to(dt).to(DEV)
    rng = np.random.default_rng(21)
    ts = [L - 1, 1500, 40, 2999]
    n_list = [300, 57, 0, 1000]
    sels = [_rand_sparse(rng, ts[b], 3, 20, n_list[b]) for b in range(B)]
    idx, nsel = _pack_idx(sels, max(n_list))
    tt = torch.tensor(ts, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(d_qk)
    o, lse = sa.sa_sparse_attn(q, kv, idx, nsel, 3, 20, scale, t=tt, v=v, d_v=d_v, return_lse=True)
    torch.cuda.synchronize()
    qf, kvf, vf = to_f64(q), to_f64(kv), to_f64(v)
    for b in range(B):
        R = O.read_set(ts[b], 3, 20, sels[b])
        oo, ol = O.sparse_attn(qf[b], kvf, R, scale, d_qk, d_v, v=vf)
        np.testing.assert_allclose(o[b].double().cpu().numpy(), oo, atol=tol, rtol=0)
        np.testing.assert_allclose(lse[b].double().cpu().numpy(), ol, atol=max(tol, 1e-4), rtol=0)
