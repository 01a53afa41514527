"""Capture of the entry points in a HIP graph: the library launches only kernels (no memset, no host
synchronisation, no allocation), so a captured step replays to the eager result. Each graph is replayed several
times, with fresh garbage in the workspace and outputs and eager work and synchronisations between the replays."""
import pytest
import torch

import long_context_sparse_sa_amd as sa
from sa_workloads import gen, get_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _check_replays(step, outs, wss):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for o in outs:
            o.fill_(-3 if o.dtype == torch.int32 else 7)
        for w in wss:
            w.fill_(0x5A + r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), r
        step()                      # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("algo", [sa.SA_TOPK_RADIX, sa.SA_TOPK_PER_QUERY, sa.SA_TOPK_RADIX_LEVELS])
def test_select_and_attention_replay(algo):
    wl = get_workload("dsa_decode_128k", L=24576, B=8)
    inp = gen.make_inputs(wl, device=DEV, seed=3)
    qd = sa.api._dtype(inp["q_idx"])
    sel_ws = torch.empty(sa.sa_select_topk_workspace(wl.L, wl.B, wl.H_I, wl.d_I, qd, qd, wl.k_sparse, algo),
                         dtype=torch.uint8, device=DEV)
    max_rows = wl.n_sink + wl.n_window + wl.k_sparse
    attn_ws = torch.empty(max(sa.sa_sparse_attn_workspace(wl.B, wl.H, wl.d_qk, wl.d_v, max_rows, sa.SA_BF16), 256),
                          dtype=torch.uint8, device=DEV)
    idx = torch.empty((wl.B, wl.k_sparse), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((wl.B,), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.B, wl.H, wl.d_v), dtype=torch.bfloat16, device=DEV)

    def step():
        sa.sa_select_topk(inp["q_idx"], inp["w"], inp["k_idx"], wl.k_sparse, wl.n_sink, wl.n_window, algo=algo,
                          ws=sel_ws, out=(idx, n_sel))
        sa.sa_sparse_attn(inp["q"], inp["kv"], idx, n_sel, wl.n_sink, wl.n_window, wl.softmax_scale, d_v=wl.d_v,
                          ws=attn_ws, out=out)

    _check_replays(step, [idx, n_sel, out], [sel_ws, attn_ws])


def test_bucket_select_replay():
    wl = get_workload("lsa_flat_1m", L=60000, n_buckets=1000, B=4)
    inp = gen.make_inputs(wl, device=DEV, seed=4, parts=("index",))
    reps, offsets, members = sa.sa_bucket_build(inp["k_idx"], inp["assign"], wl.n_buckets)
    lib = sa.api._lib.load()
    ws = torch.empty(lib.sa_bucket_select_workspace(wl.B, wl.n_buckets, 32), dtype=torch.uint8, device=DEV)
    cap = 4096
    idx = torch.empty((wl.B, cap), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((wl.B,), dtype=torch.int32, device=DEV)

    def step():
        st = lib.sa_bucket_select(inp["q_idx"].data_ptr(), sa.api._dtype(inp["q_idx"]), wl.B, wl.d_I,
                                  reps.data_ptr(), offsets.data_ptr(), members.data_ptr(), wl.n_buckets, wl.L, None,
                                  32, 4, 128, idx.data_ptr(), cap, n_sel.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                  torch.cuda.current_stream().cuda_stream)
        sa.api._lib.check("sa_bucket_select", st)

    _check_replays(step, [idx, n_sel], [ws])
