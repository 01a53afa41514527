"""The C ABI boundary without a GPU: the library loads, exports every symbol include/sa.h declares, sizes its
workspaces on the host, and rejects bad arguments before any HIP call (fake device pointers are never touched)."""
import os
import re

import pytest

from long_context_sparse_sa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, DTYPE, ALIGN, WS, UNSUP = 0, 1, 2, 3, 4, 5, 6
F32, BF16, E4M3 = 0, 1, 2
A = 0x10000          # a 16-byte aligned fake device address: validation must reject before dereferencing
MIS = 0x10008        # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "sa.h")).read()
    return re.findall(r"SA_API\s+[\w\s\*]+?\b(sa_\w+)\s*\(", text)


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_symbols()
    assert len(names) == 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings(lib):
    assert lib.sa_status_string(0) == b"SA_OK"
    assert lib.sa_status_string(5) == b"SA_ERR_WORKSPACE"
    assert lib.sa_version() == 1


def idx_score(lib, **kw):
    a = dict(q=A, qd=BF16, w=A, k=A, kd=BF16, k_ld=128, L=1024, B=2, H=64, d=128, t=None, s0=0, s1=1024, out=A,
             ld=1024)
    a.update(kw)
    return lib.sa_index_score(a["q"], a["qd"], a["w"], a["k"], a["kd"], a["k_ld"], a["L"], a["B"], a["H"], a["d"],
                              a["t"], a["s0"], a["s1"], a["out"], a["ld"], None)


def test_index_score_validation(lib):
    assert idx_score(lib, q=None) == NULL
    assert idx_score(lib, out=None) == NULL
    assert idx_score(lib, qd=7) == DTYPE
    assert idx_score(lib, qd=F32) == DTYPE                 # q and k dtypes must match
    assert idx_score(lib, k_ld=64) == SHAPE
    assert idx_score(lib, s1=2048) == SHAPE
    assert idx_score(lib, s0=10, s1=5) == SHAPE
    assert idx_score(lib, ld=10) == SHAPE
    assert idx_score(lib, L=0) == SHAPE
    assert idx_score(lib, q=MIS) == ALIGN
    assert idx_score(lib, k_ld=132) == ALIGN               # 264-byte rows are not 16-byte multiples
    assert idx_score(lib, d=100, k_ld=128) == ALIGN
    assert idx_score(lib, B=0) == OK                       # nothing to do: no launch
    assert "s_begin" in lib.sa_last_error().decode() or True


def topk(lib, **kw):
    a = dict(q=A, qd=BF16, w=A, k=A, kd=BF16, k_ld=128, L=131072, B=16, H=64, d=128, t=None, kk=2048, ns=0, nw=0,
             idx=A, idx_ld=2048, nsel=A, ws=A, wsb=0, algo=0)
    a.update(kw)
    return lib.sa_select_topk(a["q"], a["qd"], a["w"], a["k"], a["kd"], a["k_ld"], a["L"], a["B"], a["H"], a["d"],
                              a["t"], a["kk"], a["ns"], a["nw"], a["idx"], a["idx_ld"], a["nsel"], a["ws"], a["wsb"],
                              a["algo"], None)


def test_select_topk_validation(lib):
    assert topk(lib, idx=None) == NULL
    assert topk(lib, kk=0) == SHAPE
    assert topk(lib, kk=20000, idx_ld=20000) == SHAPE
    assert topk(lib, idx_ld=100) == SHAPE
    assert topk(lib, ns=-1) == SHAPE
    assert topk(lib, algo=9) == SHAPE
    assert topk(lib, ws=None) == WS
    assert topk(lib, wsb=100) == WS
    assert topk(lib, qd=F32, kd=F32, k_ld=128, d=128, algo=2) == UNSUP   # per-query streaming needs the MFMA shapes
    assert topk(lib, H=48, algo=2) == UNSUP
    need = lib.sa_select_topk_workspace(131072, 16, 64, 128, BF16, BF16, 2048, 0)
    assert need > 0
    assert topk(lib, wsb=need - 1) == WS
    assert topk(lib, ws=MIS, wsb=need) == ALIGN
    assert topk(lib, B=0, wsb=need) == OK


def test_select_topk_workspace_sizes(lib):
    # split-L decode at 128K: 2 levels, the larger covers 114688 positions
    s = lib.sa_select_topk_workspace(131072, 16, 64, 128, BF16, BF16, 2048, 1)
    assert 2 * 16 * 114688 * 8 < s < 4 * 16 * 114688 * 8
    # the per-query algorithm keeps ~2k candidates per query, twice (buffer and merge gather)
    p = lib.sa_select_topk_workspace(131072, 32768, 64, 128, BF16, BF16, 2048, 2)
    assert p >= 2 * 32768 * 4160 * 8
    assert lib.sa_select_topk_workspace(131072, 32768, 64, 128, BF16, BF16, 2048, 0) == p  # AUTO picks per-query
    assert lib.sa_select_topk_workspace(0, 1, 1, 1, F32, F32, 1, 0) == 0


def test_select_topk_auto_choices(lib):
    # up to 2^24 keys over all queries AUTO takes the plain radix select (one key per position)
    r = lib.sa_select_topk_workspace(131072, 16, 64, 128, BF16, BF16, 2048, 3)
    assert r >= 16 * 131072 * 4
    assert lib.sa_select_topk_workspace(131072, 16, 64, 128, BF16, BF16, 2048, 0) == r
    # beyond that, the radix select over a prefix of at most 2^24 / B positions, then emission levels
    L, B = 10_000_000, 4
    w = lib.sa_select_topk_workspace(L, B, 64, 128, E4M3, E4M3, 2048, 4)
    assert lib.sa_select_topk_workspace(L, B, 64, 128, E4M3, E4M3, 2048, 0) == w
    prefix = (1 << 24) // B // 512 * 512
    assert B * prefix * 4 <= w < B * L * 4 + B * (L - prefix) * 16 + (64 << 20)
    # a cache too short to split is selected whole by the radix part
    assert lib.sa_select_topk_workspace(600, 1, 64, 128, BF16, BF16, 100, 4) > 0


def attn(lib, **kw):
    a = dict(q=A, kv=A, v=None, dt=BF16, kv_ld=576, v_ld=0, L=4096, B=2, H=128, dqk=576, dv=576, t=None, idx=A,
             idx_ld=64, nsel=A, ns=4, nw=8, scale=0.04, out=A, lse=None, ws=A, wsb=1 << 30)
    a.update(kw)
    return lib.sa_sparse_attn(a["q"], a["kv"], a["v"], a["dt"], a["kv_ld"], a["v_ld"], a["L"], a["B"], a["H"],
                              a["dqk"], a["dv"], a["t"], a["idx"], a["idx_ld"], a["nsel"], a["ns"], a["nw"],
                              a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], None)


def test_sparse_attn_validation(lib):
    assert attn(lib, q=None) == NULL
    assert attn(lib, nsel=None) == NULL                   # idx and n_sel go together
    assert attn(lib, dt=E4M3) == DTYPE
    assert attn(lib, kv_ld=500) == SHAPE
    assert attn(lib, dv=2048, kv_ld=4096, dqk=576) == SHAPE
    assert attn(lib, scale=float("inf")) == SHAPE
    assert attn(lib, ns=-2) == SHAPE
    assert attn(lib, q=MIS) == ALIGN
    assert attn(lib, ws=None) == WS
    assert attn(lib, wsb=16) == WS
    assert attn(lib, B=0) == OK


def test_sparse_attn_workspace(lib):
    assert lib.sa_sparse_attn_workspace(16, 128, 576, 576, 2048, BF16) > 0     # split-K partials on the MFMA path
    assert lib.sa_sparse_attn_workspace(1, 1, 64, 64, 100, F32) == 0           # generic path: no workspace
    # the bound never shrinks as the read-set bound grows
    prev = 0
    for rows in range(32, 20000, 97):
        cur = lib.sa_sparse_attn_workspace(16, 128, 576, 576, rows, BF16)
        assert cur >= prev
        prev = cur


def test_bucket_validation(lib):
    nb = 16384
    need_b = lib.sa_bucket_build_workspace(1 << 20, nb)
    assert need_b >= 4 * nb
    assert lib.sa_bucket_build(None, BF16, 128, 1 << 20, 128, A, nb, A, A, A, A, need_b, None) == NULL
    assert lib.sa_bucket_build(A, E4M3, 128, 1 << 20, 128, A, nb, A, A, A, A, need_b, None) == DTYPE
    assert lib.sa_bucket_build(A, BF16, 128, 1 << 20, 128, A, nb, A, A, A, A, need_b - 1, None) == WS
    need_s = lib.sa_bucket_select_workspace(8, nb, 32)
    args = [A, BF16, 8, 128, A, A, A, nb, 1 << 20, None, 32, 4, 128, A, 8192, A, None, A, need_s, None]
    assert lib.sa_bucket_select(*args[:13], None, *args[14:]) == NULL
    bad = list(args); bad[10] = 0
    assert lib.sa_bucket_select(*bad) == SHAPE
    bad = list(args); bad[10] = 2000
    assert lib.sa_bucket_select(*bad) == SHAPE
    bad = list(args); bad[14] = 100000
    assert lib.sa_bucket_select(*bad) == SHAPE
    bad = list(args); bad[18] = need_s - 1
    assert lib.sa_bucket_select(*bad) == WS
    bad = list(args); bad[2] = 0
    assert lib.sa_bucket_select(*bad) == OK
