"""GPU parity of the block-granular indexers against the oracle ("long-context attention" lecture: sections "Qwen
Sparse Attention" and "MiniMax Sparse Attention").

* QSA: pooled keys bit-exact; integer-valued inputs make every pooled key and score exact, so the read sets must
  match bit for bit (ties to the lower micro-block); normal inputs compare the chosen micro-blocks outside the band
  of blocks whose fp32 score lies within 1e-5 relative of the k-th block score, and the tail exactly.
* MSA: integer-valued inputs exact per (query, group); normal inputs band-compare the chosen earlier blocks at the
  (k_b - 1)-th block score, and the local block exactly.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_sa_amd as sa
from oracle import sa_oracle as O
from tests.gpu_helpers import band_compare, selected, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
DT = {"bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}


def _inputs(seed, B, H, d, L, integer, dtype="bf16"):
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


# ---------------------------------------------------------------------------------------------------------- QSA
def test_qsa_pool_bit_exact():
    _, _, k = _inputs(1, 1, 1, 128, 10_003, integer=False)
    pooled = sa.sa_qsa_pool(k, 4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_f64(pooled), O.qsa_pool(to_f64(k), 4))


def _qsa_parts(pos, t, b):
    """Split an expanded QSA read set into (chosen micro-blocks, tail positions)."""
    n_complete = (t + 1) // b
    tail_n = t + 1 - n_complete * b
    body, tail = pos[:pos.size - tail_n], pos[pos.size - tail_n:]
    assert body.size % b == 0
    blocks = body[::b] // b
    np.testing.assert_array_equal(body, (blocks[:, None] * b + np.arange(b)[None, :]).reshape(-1))
    return blocks, tail


@pytest.mark.parametrize("H", [64, 32])
def test_qsa_integer_exact_with_ties(H):
    B, L, b, kb = 7, 40_000, 4, 300
    q, w, k = _inputs(2, B, H, 128, L, integer=True)
    ts = [L - 1, 39_998, 20_001, 1_000, 3, 2, 0]
    tt = torch.tensor(ts, dtype=torch.int32, device=DEV)
    pooled = sa.sa_qsa_pool(k, b)
    idx, n_sel = sa.sa_qsa_select(q, w, pooled, L, b, kb, t=tt)
    torch.cuda.synchronize()
    qf, wf, pf = to_f64(q), w.double().cpu().numpy(), to_f64(pooled)
    for i in range(B):
        ref, _, _ = O.qsa_select(qf[i], wf[i], pf, ts[i], b, kb)
        np.testing.assert_array_equal(selected(idx[i], int(n_sel[i].item())), ref)


def test_qsa_normal_decode_release_budget():
    # 2048 tokens of micro-blocks of 4: 512 blocks per query
    B, L, b, kb = 5, 131_072, 4, 512
    q, w, k = _inputs(3, B, 64, 128, L, integer=False)
    pooled = sa.sa_qsa_pool(k, b)
    ts = [L - 1, L - 2, 100_001, 77_778, 4_099]
    tt = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, n_sel = sa.sa_qsa_select(q, w, pooled, L, b, kb, t=tt)
    torch.cuda.synchronize()
    qf, wf, pf = to_f64(q), w.double().cpu().numpy(), to_f64(pooled)
    for i in range(B):
        ref, ref_blocks, sc = O.qsa_select(qf[i], wf[i], pf, ts[i], b, kb)
        got = selected(idx[i], int(n_sel[i].item()))
        blocks, tail = _qsa_parts(got, ts[i], b)
        _, ref_tail = _qsa_parts(ref, ts[i], b)
        np.testing.assert_array_equal(tail, ref_tail)
        band_compare(blocks, ref_blocks, np.arange(sc.size), sc, kb)


# ---------------------------------------------------------------------------------------------------------- MSA
@pytest.mark.parametrize("dtype,G", [("bf16", 2), ("bf16", 1), ("e4m3", 2)])
def test_msa_integer_exact_with_ties(dtype, G):
    B, H, L, c, kb = 5, 64, 20_000, 128, 16
    q, w, k = _inputs(4, B, H, 128, L, integer=True, dtype=dtype)
    ts = [L - 1, 12_345, 128, 127, 5]
    tt = torch.tensor(ts, dtype=torch.int32, device=DEV)
    idx, n_sel = sa.sa_msa_select(q, w, k, G, c, kb, t=tt)
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for i in range(B):
        res = O.msa_select(qf[i], wf[i], kf, ts[i], G, c, kb)
        for g in range(G):
            np.testing.assert_array_equal(selected(idx[i * G + g], int(n_sel[i * G + g].item())), res[g][0])


def test_msa_local_block_only():
    B, H, L, c = 3, 64, 5000, 128
    q, w, k = _inputs(5, B, H, 128, L, integer=False)
    ts = [L - 1, 300, 64]
    idx, n_sel = sa.sa_msa_select(q, w, k, 2, c, 1, t=torch.tensor(ts, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for i in range(B):
        for g in range(2):
            np.testing.assert_array_equal(selected(idx[i * 2 + g], int(n_sel[i * 2 + g].item())),
                                          np.arange(ts[i] // c * c, ts[i] + 1))


def test_msa_normal_prefill_chunk():
    """Causal chunk: 32 consecutive queries at the end of a 256K cache, two groups of 32 indexer heads, 16 blocks of
    128 per group (the lecture's per-group budget of 2048 positions)."""
    B, H, L, c, kb, G = 32, 64, 262_144, 128, 16, 2
    q, w, k = _inputs(6, B, H, 128, L, integer=False)
    ts = list(range(L - B, L))
    idx, n_sel = sa.sa_msa_select(q, w, k, G, c, kb, t=torch.tensor(ts, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    qf, wf, kf = to_f64(q), w.double().cpu().numpy(), to_f64(k)
    for i in (0, 13, 31):
        res = O.msa_select(qf[i], wf[i], kf, ts[i], G, c, kb)
        for g in range(G):
            pos, blocks, bsc = res[g]
            got = selected(idx[i * G + g], int(n_sel[i * G + g].item()))
            local = ts[i] // c
            np.testing.assert_array_equal(got[got >= local * c], np.arange(local * c, ts[i] + 1))
            body = got[got < local * c]
            got_blocks = body[::c] // c
            np.testing.assert_array_equal(body, (got_blocks[:, None] * c + np.arange(c)[None, :]).reshape(-1))
            band_compare(got_blocks, blocks[:-1], np.arange(local), bsc, kb - 1)
