"""GPU parity of sa_index_score and sa_select_topk against the oracle (LongCat deep-dive: DSA baseline section,
indexer and arg-topK equations; SI section, top-K over positions outside sink and window).

Integer-valued inputs make every score exact, so the selected sets must match bit for bit, ties included.
Normal inputs compare outside the band of positions whose fp32 score lies within 1e-5 relative of the k-th score.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from tests.gpu_helpers import band_compare, selected, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}


def _inputs(seed, B, H, d, L, dtype, integer):
    g = torch.Generator(device="cpu").manual_seed(seed)
    if integer:
        q = torch.randint(-2, 3, (B, H, d), generator=g).float()
        k = torch.randint(-2, 3, (L, d), generator=g).float()
        w = torch.randint(0, 3, (B, H), generator=g).float()
    else:
        q = torch.randn((B, H, d), generator=g)
        k = torch.randn((L, d), generator=g)
        w = torch.randn((B, H), generator=g)
    return q.to(DT[dtype]).to(DEV), w.to(DEV), k.to(DT[dtype]).to(DEV)


@pytest.mark.parametrize("dtype,H,d", [("bf16", 64, 128), ("bf16", 32, 128), ("e4m3", 64, 128), ("f32", 4, 32),
                                       ("bf16", 3, 16)])
def test_index_score_dense(dtype, H, d):
    B, L = 5, 3000
    q, w, k = _inputs(11, B, H, d, L, dtype, integer=False)
    t = torch.tensor([L - 1, 100, 2999, 0, 1500], dtype=torch.int32, device=DEV)
    s0, s1 = 37, 2900
    sc = sa.sa_index_score(q, w, k, t=t, s_begin=s0, s_end=s1)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    got = sc.cpu().numpy()
    for b in range(B):
        pos = np.arange(s0, s1)
        ref = O.index_score(qf[b], wf[b], kf, pos)
        mag = np.abs(kf[pos] @ np.abs(qf[b]).T) @ np.abs(wf[b])      # bound on the magnitude of the summed terms
        vis = pos <= t[b].item()
        assert np.all(np.isneginf(got[b][~vis]))
        err = np.abs(got[b][vis] - ref[vis])
        assert np.all(err <= 1e-5 * mag[vis] + 1e-30), (b, err.max())


ALGOS = [sa.SA_TOPK_SPLIT_L, sa.SA_TOPK_PER_QUERY, sa.SA_TOPK_RADIX, sa.SA_TOPK_RADIX_LEVELS, sa.SA_TOPK_STREAM]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("B", [6, 9])
def test_topk_integer_exact_with_ties(algo, dtype, B):
    """Integer-valued q, k in {-2..2} and w in {0,1,2}: scores are exact, selection must match bit for bit.
    B = 6 runs 4-query workgroups; B = 9 runs 8-query workgroups with a partly empty second group in the dense and
    emitting scorer, and three 4-query workgroups (the last partly empty) in the streaming select."""
    H, d, L, kk = 64, 128, 40000, 700
    q, w, k = _inputs(5, B, H, d, L, dtype, integer=True)
    ts = ([L - 1, 39000, 20000, 17000, 5000, 900, 33333, 123, 39999])[:B]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=3, n_window=50, t=t, algo=algo)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 3, 50)
        if b == 0:
            assert np.unique(sc).size < sc.size / 4        # heavy ties are really exercised
        got = selected(idx[b], nsel[b].item())
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_topk_stream_eight_query_groups(dtype):
    """The streaming select takes 8-query workgroups from 32 queries up: B = 33 leaves one query in the last group.
    Integer inputs, exact scores, bit-exact selection."""
    B, H, d, L, kk = 33, 64, 128, 6000, 300
    q, w, k = _inputs(21, B, H, d, L, dtype, integer=True)
    ts = [L - 1 - 97 * b for b in range(B)]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=2, n_window=30, t=t, algo=sa.SA_TOPK_STREAM)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 2, 30)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)


@pytest.mark.parametrize("algo", ALGOS)
def test_topk_heads32_integer_exact(algo):
    """32 indexer heads (one head tile per query wave): integer inputs, exact scores, bit-exact selection."""
    B, H, d, L, kk = 5, 32, 128, 30000, 500
    q, w, k = _inputs(15, B, H, d, L, "bf16", integer=True)
    ts = [L - 1, 29000, 12000, 700, 20001]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=2, n_window=40, t=t, algo=algo)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 2, 40)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)


@pytest.mark.parametrize("algo", [sa.SA_TOPK_RADIX, sa.SA_TOPK_RADIX_LEVELS, sa.SA_TOPK_SPLIT_L, sa.SA_TOPK_STREAM])
def test_topk_single_query(algo):
    """B = 1: the radix select spreads one query over its largest number of chunks."""
    B, H, d, L, kk = 1, 64, 128, 200000, 1000
    q, w, k = _inputs(16, B, H, d, L, "bf16", integer=True)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=1, n_window=16, algo=algo)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    ref, sc, cand = O.select_topk(qf[0], wf[0], kf, L - 1, kk, 1, 16)
    np.testing.assert_array_equal(selected(idx[0], nsel[0].item()), ref)


@pytest.mark.parametrize("algo", ALGOS)
def test_topk_normal_band(algo):
    B, H, d, L, kk = 8, 64, 128, 150000, 2048
    q, w, k = _inputs(7, B, H, d, L, "bf16", integer=False)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=4, n_window=128, algo=algo)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in (0, 3, 7):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, L - 1, kk, 4, 128)
        band_compare(selected(idx[b], nsel[b].item()), ref, cand, sc, kk)


@pytest.mark.parametrize("algo", [sa.SA_TOPK_SPLIT_L, sa.SA_TOPK_RADIX, sa.SA_TOPK_RADIX_LEVELS])
def test_topk_valu_path_f32(algo):
    """The toy indexer shapes (4 heads x 32, fp32) take the VALU scorer."""
    B, H, d, L, kk = 2, 4, 32, 1024, 64
    q, w, k = _inputs(3, B, H, d, L, "f32", integer=False)
    w = w.abs()
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=4, n_window=32, algo=algo)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, L - 1, kk, 4, 32)
        band_compare(selected(idx[b], nsel[b].item()), ref, cand, sc, kk)


@pytest.mark.parametrize("algo", ALGOS)
def test_topk_degenerate(algo):
    """k larger than the candidate set, k = 1, and queries whose sink and window cover every visible position."""
    B, H, d, L = 4, 64, 128, 3000
    q, w, k = _inputs(9, B, H, d, L, "bf16", integer=True)
    ts = [2999, 10, 1, 600]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for kk in (1, 5000):
        idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=4, n_window=8, t=t, algo=algo, idx_ld=kk + 3)
        torch.cuda.synchronize()
        for b in range(B):
            ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 4, 8)
            np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)


def test_topk_all_equal_scores():
    """Every score equal: the lowest candidate positions win."""
    B, H, d, L, kk = 2, 64, 128, 20000, 300
    q = torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV)
    w = torch.ones((B, H), device=DEV)
    k = torch.ones((L, d), dtype=torch.bfloat16, device=DEV)
    for algo in ALGOS:
        idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=2, n_window=3, algo=algo)
        torch.cuda.synchronize()
        for b in range(B):
            np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), np.arange(2, 2 + kk))


def test_topk_valu_path_levels():
    """VALU scorer (4 heads x 32, fp32) over two key ranges: the second range emits into per-workgroup segments."""
    B, H, d, L, kk = 3, 4, 32, 40000, 300
    q, w, k = _inputs(13, B, H, d, L, "f32", integer=False)
    ts = [L - 1, 30000, 17000]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=2, n_window=16, t=t, algo=sa.SA_TOPK_SPLIT_L)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 2, 16)
        band_compare(selected(idx[b], nsel[b].item()), ref, cand, sc, kk)


@pytest.mark.parametrize("algo", [sa.SA_TOPK_SPLIT_L, sa.SA_TOPK_RADIX_LEVELS, sa.SA_TOPK_STREAM])
def test_topk_rising_scores_many_emits(algo):
    """Scores rise with position (with runs of equal bf16 keys): every later key range emits almost all of its
    positions, so the merges overflow LDS and run from the gather buffer; ties resolve to lower positions."""
    B, H, d, L, kk = 2, 64, 128, 150000, 2048
    k = torch.zeros((L, d), dtype=torch.float32)
    k[:, 0] = torch.arange(L, dtype=torch.float32) / 1000.0
    k = k.to(torch.bfloat16).to(DEV)
    q = torch.zeros((B, H, d), dtype=torch.float32)
    q[:, :, 0] = 1.0
    q[1, :, 1] = 0.5
    q = q.to(torch.bfloat16).to(DEV)
    w = torch.ones((B, H), device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=4, n_window=64, algo=algo)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, L - 1, kk, 4, 64)
        assert np.unique(sc).size < sc.size  # ties are exercised
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)


def test_topk_radix_chunks_and_ties():
    """Radix select over many chunks per query: integer scores tie heavily, so the k-th key is shared by entries of
    several chunks and the lowest positions must win across chunk boundaries; one query has fewer candidates than
    k (every candidate is kept, -1 padding after them)."""
    B, H, d, L, kk = 3, 64, 128, 100000, 3000
    q, w, k = _inputs(11, B, H, d, L, "bf16", integer=True)
    ts = [L - 1, 60001, 2500]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=5, n_window=40, t=t, algo=sa.SA_TOPK_RADIX, idx_ld=kk + 17)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(B):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, 5, 40)
        if b == 0:
            assert np.unique(sc).size < sc.size / 4
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)
    assert nsel[2].item() == 2500 - 5 - 40 + 1


@pytest.mark.parametrize("algo", ALGOS + [sa.SA_TOPK_AUTO])
def test_topk_prefilled_workspace_and_outputs(algo):
    """Whatever the workspace and the output buffers hold before the call (all-ones bytes, a byte pattern, zeros),
    the selection is the same exact result: the kernels clear every counter, histogram and record they use, and idx
    is overwritten in full, padding included. The calls run back to back on one workspace."""
    B, H, d, L, kk, ld = 6, 64, 128, 40000, 700, 711
    q, w, k = _inputs(5, B, H, d, L, "bf16", integer=True)
    ts = [L - 1, 39000, 20000, 17000, 5000, 300]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    nbytes = sa.sa_select_topk_workspace(L, B, H, d, sa.SA_BF16, sa.SA_BF16, kk, algo)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    refs = [O.select_topk(qf[b], wf[b], kf, ts[b], kk, 3, 50)[0] for b in range(B)]
    for fill in (0xFF, 0x5A, 0x00):
        ws.fill_(fill)
        idx = torch.full((B, ld), -7, dtype=torch.int32, device=DEV)
        nsel = torch.full((B,), 12345, dtype=torch.int32, device=DEV)
        sa.sa_select_topk(q, w, k, kk, n_sink=3, n_window=50, t=t, algo=algo, idx_ld=ld, ws=ws, out=(idx, nsel))
        torch.cuda.synchronize()
        for b in range(B):
            n = nsel[b].item()
            assert n == refs[b].size, (fill, b, n)
            np.testing.assert_array_equal(selected(idx[b], n), refs[b])
            assert torch.all(idx[b, n:] == -1), (fill, b)


def _exact_check(q, w, k, kk, n_sink, n_window, ts, idx, nsel):
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for b in range(q.shape[0]):
        ref, sc, cand = O.select_topk(qf[b], wf[b], kf, ts[b], kk, n_sink, n_window)
        np.testing.assert_array_equal(selected(idx[b], nsel[b].item()), ref)


@pytest.mark.parametrize("spin", [0, 1])
def test_topk_stream_bound_without_waiting(spin):
    """The streaming select with its wait cut to `spin` polls (a test knob set from the host): workgroups go on with
    whatever statistics are published by then, so their bounds are weaker and more keys reach the merge, but the
    selection is the same. Integer scores (exact, heavy ties), three launches of 16 queries, per-query t."""
    B, H, d, L, kk = 16, 64, 128, 300000, 2048
    q, w, k = _inputs(21, B, H, d, L, "bf16", integer=True)
    ts = [L - 1 - 7919 * b for b in range(B)]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    lib = sa.load()
    lib.sa_set_stream_spin_limit(spin)
    try:
        idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=4, n_window=128, t=t, algo=sa.SA_TOPK_STREAM)
        torch.cuda.synchronize()
    finally:
        lib.sa_set_stream_spin_limit(-1)
    _exact_check(q, w, k, kk, 4, 128, ts, idx, nsel)


def test_topk_stream_launches_carry_the_bound_fp8():
    """Few queries (four per workgroup) over more positions than one launch's resident workgroups cover: later
    launches start from the bound of the earlier ones. e4m3 integer inputs: exact scores."""
    B, H, d, L, kk = 3, 64, 128, 1_300_000, 2048
    q, w, k = _inputs(22, B, H, d, L, "e4m3", integer=True)
    ts = [L - 1, L - 1 - 250_000, 700_000]
    t = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=4, n_window=128, t=t, algo=sa.SA_TOPK_STREAM)
    torch.cuda.synchronize()
    _exact_check(q, w, k, kk, 4, 128, ts, idx, nsel)


def test_topk_stream_repeated_calls_one_workspace():
    """Calls in a row on one workspace with different data: the statistics slots of a call are cleared by its merge
    and tagged with the call's nonce, so no call sees another's."""
    B, H, d, L, kk = 9, 64, 128, 140000, 1000
    ws = None
    for seed in (30, 31, 32):
        q, w, k = _inputs(seed, B, H, d, L, "bf16", integer=True)
        if ws is None:
            ws = torch.empty(sa.sa_select_topk_workspace(L, B, H, d, sa.SA_BF16, sa.SA_BF16, kk, sa.SA_TOPK_STREAM),
                             dtype=torch.uint8, device=DEV)
        idx, nsel = sa.sa_select_topk(q, w, k, kk, n_sink=2, n_window=16, algo=sa.SA_TOPK_STREAM, ws=ws)
        torch.cuda.synchronize()
        _exact_check(q, w, k, kk, 2, 16, [L - 1] * B, idx, nsel)
