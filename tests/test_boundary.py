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
    assert sorted(names) == sorted(_lib.SIGNATURES)
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
    # few queries on the MFMA scorer shapes: AUTO takes the streaming algorithm (5), whose workspace reserves, for
    # the first min(L, 2^20) positions scored on chip, one 8-byte candidate slot per position for the emitted
    # segments and as many for the merge's overflow (only candidates at or above the bound are ever written), plus
    # per-workgroup statistics; beyond 2^20 positions, the emission levels' candidate areas
    for L, B, dt in [(131072, 16, BF16), (10_000_000, 4, E4M3), (1000, 1, BF16)]:
        s = lib.sa_select_topk_workspace(L, B, 64, 128, dt, dt, 2048, 5)
        assert lib.sa_select_topk_workspace(L, B, 64, 128, dt, dt, 2048, 0) == s
        first = min(L, 1 << 20)
        assert B * first * 16 <= s
        if L <= 1 << 20:
            assert s < B * (L + 2048) * 16 + B * (L // 512 + 2) * 12 + B * 1025 * 4 + (1 << 20)
        else:
            assert s < B * L * 16 + (64 << 20)
    # many queries: the per-query streaming select (2)
    assert lib.sa_select_topk_workspace(131072, 64, 64, 128, BF16, BF16, 2048, 0) == \
        lib.sa_select_topk_workspace(131072, 64, 64, 128, BF16, BF16, 2048, 2)
    # shapes the MFMA scorer does not serve (fp32 here): the radix select over one key per position up to 2^24
    # keys over all queries ...
    r = lib.sa_select_topk_workspace(131072, 16, 64, 128, F32, F32, 2048, 3)
    assert r >= 16 * 131072 * 4
    assert lib.sa_select_topk_workspace(131072, 16, 64, 128, F32, F32, 2048, 0) == r
    # ... and beyond that the radix select over a prefix of at most 2^24 / B positions, then emission levels
    L, B = 10_000_000, 4
    w = lib.sa_select_topk_workspace(L, B, 4, 32, F32, F32, 2048, 4)
    assert lib.sa_select_topk_workspace(L, B, 4, 32, F32, F32, 2048, 0) == w
    prefix = (1 << 24) // B // 256 * 256
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


def test_bucket_select_noalloc_validation(lib):
    """The no-allocation variant validates like the workspace variant and rejects, before any HIP call, calls
    whose keys do not fit its static scratch array."""
    max_keys = lib.sa_bucket_select_noalloc_max_keys()
    assert max_keys == 1 << 21
    nb = 1 << 17
    args = [A, BF16, max_keys // nb, 128, A, A, A, nb, 1 << 20, None, 32, 4, 128, A, 8192, A, None, None]
    assert lib.sa_bucket_select_noalloc(*args[:13], None, *args[14:]) == NULL
    bad = list(args); bad[1] = E4M3
    assert lib.sa_bucket_select_noalloc(*bad) == DTYPE
    bad = list(args); bad[10] = 0
    assert lib.sa_bucket_select_noalloc(*bad) == SHAPE
    bad = list(args); bad[2] = max_keys // nb + 1
    assert lib.sa_bucket_select_noalloc(*bad) == WS
    assert b"static scratch" in lib.sa_last_error()
    bad = list(args); bad[2] = 0
    assert lib.sa_bucket_select_noalloc(*bad) == OK  # nothing to do: no HIP call


def hi(lib, **kw):
    a = dict(q=A, qd=BF16, w=A, k=A, kd=BF16, k_ld=128, L=131072, B=4, H=64, d=128, t=None, means=A, sub=8, P=128,
             M=64, kk=2048, ns=4, nw=128, idx=A, idx_ld=2048, nsel=A, pages=None, ws=A, wsb=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = lib.sa_hi_select_workspace(a["L"], a["B"], a["sub"], a["P"], a["M"], a["kk"])
    return lib.sa_hi_select(a["q"], a["qd"], a["w"], a["k"], a["kd"], a["k_ld"], a["L"], a["B"], a["H"], a["d"],
                            a["t"], a["means"], a["sub"], a["P"], a["M"], a["kk"], a["ns"], a["nw"], a["idx"],
                            a["idx_ld"], a["nsel"], a["pages"], a["ws"], a["wsb"], None)


def test_hi_validation(lib):
    assert hi(lib, means=None) == NULL
    assert hi(lib, idx=None) == NULL
    assert hi(lib, qd=E4M3, kd=E4M3) == UNSUP          # the token stage reads bf16 keys
    assert hi(lib, H=48) == UNSUP
    assert hi(lib, P=96) == SHAPE                      # pages are whole 64-position tiles
    assert hi(lib, P=128, sub=3) == SHAPE              # sub-blocks tile the page
    assert hi(lib, P=128, sub=1) == SHAPE              # 128 sub-blocks per page: more than one tile of means
    assert hi(lib, M=0) == SHAPE
    assert hi(lib, M=(1 << 20) + 1) == SHAPE
    assert hi(lib, kk=0) == SHAPE
    assert hi(lib, idx_ld=100) == SHAPE
    assert hi(lib, means=MIS) == ALIGN
    assert hi(lib, ws=None) == WS
    need = lib.sa_hi_select_workspace(131072, 4, 8, 128, 64, 2048)
    assert hi(lib, wsb=need - 1) == WS
    assert hi(lib, B=0) == OK
    # the workspace holds the page scores, the page select's keys and the token stage's buffers
    assert need >= 4 * 1024 * 4 * 2 + 2 * 4 * (4 * 2048 + 64) * 8
    assert lib.sa_hi_build(None, BF16, 128, 1000, 128, 8, A, None) == NULL
    assert lib.sa_hi_build(A, E4M3, 128, 1000, 128, 8, A, None) == DTYPE
    assert lib.sa_hi_build(A, BF16, 64, 1000, 128, 8, A, None) == SHAPE
    assert lib.sa_hi_build(A, BF16, 128, 1000, 128, 0, A, None) == SHAPE


def test_qsa_msa_validation(lib):
    B, H, d, L = 4, 64, 128, 100_000
    need_q = lib.sa_qsa_select_workspace(L, B, H, d, 4, 512)
    assert need_q > 0

    def qsa(**kw):
        a = dict(q=A, qd=BF16, w=A, pooled=A, L=L, B=B, H=H, d=d, t=None, block=4, kb=512, idx=A,
                 idx_ld=512 * 4 + 3, nsel=A, ws=A, wsb=need_q)
        a.update(kw)
        return lib.sa_qsa_select(a["q"], a["qd"], a["w"], a["pooled"], a["L"], a["B"], a["H"], a["d"], a["t"],
                                 a["block"], a["kb"], a["idx"], a["idx_ld"], a["nsel"], a["ws"], a["wsb"], None)

    assert qsa(idx=None) == NULL
    assert qsa(pooled=None) == NULL
    assert qsa(qd=E4M3) == DTYPE                   # pooled keys are bf16
    assert qsa(block=0) == SHAPE
    assert qsa(kb=0) == SHAPE
    assert qsa(idx_ld=512 * 4 + 2) == SHAPE        # the tail needs up to block - 1 more entries
    assert qsa(wsb=need_q - 1) == WS
    assert qsa(B=0, wsb=lib.sa_qsa_select_workspace(L, 0, H, d, 4, 512)) == OK

    need_m = lib.sa_msa_select_workspace(L, B, 2, 128, 16)
    assert need_m > 0

    def msa(**kw):
        a = dict(q=A, qd=BF16, w=A, k=A, kd=BF16, k_ld=d, L=L, B=B, H=H, d=d, G=2, t=None, block=128, kb=16, idx=A,
                 idx_ld=16 * 128, nsel=A, ws=A, wsb=need_m)
        a.update(kw)
        return lib.sa_msa_select(a["q"], a["qd"], a["w"], a["k"], a["kd"], a["k_ld"], a["L"], a["B"], a["H"],
                                 a["d"], a["G"], a["t"], a["block"], a["kb"], a["idx"], a["idx_ld"], a["nsel"],
                                 a["ws"], a["wsb"], None)

    assert msa(idx=None) == NULL
    assert msa(G=3) == SHAPE                       # G must divide H
    assert msa(block=100) == SHAPE
    assert msa(kb=0) == SHAPE
    assert msa(idx_ld=16 * 128 - 1) == SHAPE
    assert msa(G=4) == UNSUP                       # 16 heads per group: no MFMA scorer shape
    assert msa(wsb=need_m - 1) == WS
    assert msa(B=0) == OK


def test_bucket_tree_validation(lib):
    import ctypes
    nb, B = 4096, 8
    ln = (ctypes.c_int32 * 2)(64, 512)
    lk = (ctypes.c_int32 * 2)(8, 64)
    need = lib.sa_bucket_tree_select_workspace(B, 2, ln, lk, nb)
    assert need >= B * (64 + 512 + nb) * 4
    rp = (ctypes.c_void_p * 2)(A, A)
    cp = (ctypes.c_void_p * 2)(A, A)

    def tree(**kw):
        a = dict(q=A, qd=F32, B=B, d=128, nl=2, rp=rp, cp=cp, ln=ln, lk=lk, reps=A, off=A, mem=A, nb=nb, L=1 << 20,
                 t=None, top_b=32, ns=4, nw=128, idx=A, cap=8192, nsel=A, bo=None, ws=A, wsb=need)
        a.update(kw)
        return lib.sa_bucket_tree_select(a["q"], a["qd"], a["B"], a["d"], a["nl"], a["rp"], a["cp"], a["ln"], a["lk"],
                                         a["reps"], a["off"], a["mem"], a["nb"], a["L"], a["t"], a["top_b"], a["ns"],
                                         a["nw"], a["idx"], a["cap"], a["nsel"], a["bo"], a["ws"], a["wsb"], None)

    assert tree(nl=0) == SHAPE
    assert tree(nl=9) == SHAPE
    assert tree(rp=None) == NULL
    assert tree(rp=(ctypes.c_void_p * 2)(A, None)) == NULL
    assert tree(lk=(ctypes.c_int32 * 2)(8, 0)) == SHAPE
    assert tree(ln=(ctypes.c_int32 * 2)(0, 512)) == SHAPE
    assert tree(rp=(ctypes.c_void_p * 2)(A, MIS)) == ALIGN
    assert tree(top_b=0) == SHAPE                  # the Flat search's own checks apply
    assert tree(wsb=need - 1) == WS
    assert tree(B=0, wsb=lib.sa_bucket_tree_select_workspace(0, 2, ln, lk, nb)) == OK
