"""Thin torch-facing binding of the C ABI in include/sa.h: same names, argument marshalling only.

Every function checks dtypes, shapes and devices, allocates outputs and workspace with torch (device memory is the
caller's), and calls the HIP library on torch's current stream. No step of the method runs here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_DT = {torch.float32: _lib.SA_F32, torch.bfloat16: _lib.SA_BF16, torch.float8_e4m3fn: _lib.SA_E4M3}


def _dtype(x: torch.Tensor) -> int:
    if x.dtype not in _DT:
        raise TypeError(f"unsupported dtype {x.dtype}")
    return _DT[x.dtype]


def _ptr(x: Optional[torch.Tensor]) -> Optional[int]:
    return None if x is None else x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need_cuda(*xs):
    for x in xs:
        if x is not None and not x.is_cuda:
            raise ValueError("all tensors must live on the GPU")


def _rows(x: torch.Tensor) -> int:
    """Leading dimension (elements) of a 2-D row-major tensor whose rows may be padded."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return x.stride(0)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------------------------------------


def sa_index_score(q_idx, w, k_idx, t=None, s_begin: int = 0, s_end: Optional[int] = None, out=None, stream=None):
    """scores[b, s - s_begin] of the lightning indexer over positions [s_begin, s_end) (-inf past t_b)."""
    _need_cuda(q_idx, w, k_idx, t, out)
    B, H, d = q_idx.shape
    L = k_idx.shape[0]
    s_end = L if s_end is None else s_end
    if out is None:
        out = torch.empty((B, max(1, s_end - s_begin)), dtype=torch.float32, device=q_idx.device)
    st = _lib.load().sa_index_score(_ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_idx), _dtype(k_idx), _rows(k_idx), L,
                                    B, H, d, _ptr(t), s_begin, s_end, _ptr(out), out.stride(0), _stream(stream))
    _lib.check("sa_index_score", st)
    return out[:, : s_end - s_begin]


def sa_select_topk_workspace(L, B, H, d, q_dtype, k_dtype, k_sparse, algo=_lib.SA_TOPK_AUTO) -> int:
    return int(_lib.load().sa_select_topk_workspace(L, B, H, d, q_dtype, k_dtype, k_sparse, algo))


def sa_select_topk(q_idx, w, k_idx, k_sparse: int, n_sink: int = 0, n_window: int = 0, t=None,
                   idx_ld: Optional[int] = None, algo: int = _lib.SA_TOPK_AUTO, ws=None, out=None, stream=None):
    """(idx [B, idx_ld] ascending with -1 padding, n_sel [B]) of the top-k candidates outside sink and window."""
    _need_cuda(q_idx, w, k_idx, t)
    B, H, d = q_idx.shape
    L = k_idx.shape[0]
    idx_ld = k_sparse if idx_ld is None else idx_ld
    lib = _lib.load()
    nbytes = lib.sa_select_topk_workspace(L, B, H, d, _dtype(q_idx), _dtype(k_idx), k_sparse, algo)
    ws = _workspace(nbytes, q_idx.device, ws)
    if out is None:
        idx = torch.empty((B, idx_ld), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
    else:
        idx, n_sel = out
    st = lib.sa_select_topk(_ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_idx), _dtype(k_idx), _rows(k_idx), L, B, H, d,
                            _ptr(t), k_sparse, n_sink, n_window, _ptr(idx), idx.stride(0), _ptr(n_sel), _ptr(ws),
                            nbytes, algo, _stream(stream))
    _lib.check("sa_select_topk", st)
    return idx, n_sel


def sa_select_topk_scores(scores, k_sparse: int, n_sink: int = 0, n_window: int = 0, t=None,
                          idx_ld: Optional[int] = None, ws=None, out=None, stream=None):
    """(idx [B, idx_ld] ascending with -1 padding, n_sel [B]) of the top-k of caller-given fp32 scores [B, L]."""
    _need_cuda(scores, t)
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a 2-D fp32 tensor with unit column stride")
    B, L = scores.shape
    idx_ld = k_sparse if idx_ld is None else idx_ld
    lib = _lib.load()
    nbytes = lib.sa_select_topk_scores_workspace(L, B)
    ws = _workspace(nbytes, scores.device, ws)
    if out is None:
        idx = torch.empty((B, idx_ld), dtype=torch.int32, device=scores.device)
        n_sel = torch.empty((B,), dtype=torch.int32, device=scores.device)
    else:
        idx, n_sel = out
    st = lib.sa_select_topk_scores(_ptr(scores), scores.stride(0), L, B, _ptr(t), k_sparse, n_sink, n_window,
                                   _ptr(idx), idx.stride(0), _ptr(n_sel), _ptr(ws), nbytes, _stream(stream))
    _lib.check("sa_select_topk_scores", st)
    return idx, n_sel


def sa_bucket_build(k_idx, assign, n_buckets: int, ws=None, stream=None):
    """(reps [NB, d] fp32, offsets [NB + 1] int32, members [L] int32) of the bucket directory."""
    _need_cuda(k_idx, assign)
    L, d = k_idx.shape
    lib = _lib.load()
    nbytes = lib.sa_bucket_build_workspace(L, n_buckets)
    ws = _workspace(nbytes, k_idx.device, ws)
    reps = torch.empty((n_buckets, d), dtype=torch.float32, device=k_idx.device)
    offsets = torch.empty((n_buckets + 1,), dtype=torch.int32, device=k_idx.device)
    members = torch.empty((L,), dtype=torch.int32, device=k_idx.device)
    st = lib.sa_bucket_build(_ptr(k_idx), _dtype(k_idx), _rows(k_idx), L, d, _ptr(assign), n_buckets, _ptr(reps),
                             _ptr(offsets), _ptr(members), _ptr(ws), nbytes, _stream(stream))
    _lib.check("sa_bucket_build", st)
    return reps, offsets, members


def sa_bucket_select(q_idx, reps, offsets, members, L: int, top_b: int, n_sink: int = 0, n_window: int = 0,
                     cap: int = 8192, t=None, return_buckets: bool = False, ws=None, stream=None):
    """(idx [B, cap] ascending with -1 padding, n_sel [B] (negative: -needed on overflow)[, buckets [B, top_b]])."""
    _need_cuda(q_idx, reps, offsets, members, t)
    B, d = q_idx.shape
    nb = reps.shape[0]
    lib = _lib.load()
    nbytes = lib.sa_bucket_select_workspace(B, nb, top_b)
    ws = _workspace(nbytes, q_idx.device, ws)
    idx = torch.empty((B, cap), dtype=torch.int32, device=q_idx.device)
    n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
    buckets = torch.empty((B, top_b), dtype=torch.int32, device=q_idx.device) if return_buckets else None
    st = lib.sa_bucket_select(_ptr(q_idx), _dtype(q_idx), B, d, _ptr(reps), _ptr(offsets), _ptr(members), nb, L,
                              _ptr(t), top_b, n_sink, n_window, _ptr(idx), cap, _ptr(n_sel), _ptr(buckets), _ptr(ws),
                              nbytes, _stream(stream))
    _lib.check("sa_bucket_select", st)
    return (idx, n_sel, buckets) if return_buckets else (idx, n_sel)


def sa_bucket_tree_select(q_idx, levels, reps, offsets, members, L: int, top_b: int, n_sink: int = 0,
                          n_window: int = 0, t=None, cap: int = 8192, return_buckets=False, ws=None, out=None,
                          stream=None):
    """Tree search over a cluster tree. levels: list, root first, of (reps_l [n_l, d] fp32, child_off_l [n_l + 1]
    int32, keep_l). Returns (idx [B, cap], n_sel [B][, buckets [B, top_b]]) as sa_bucket_select."""
    import ctypes
    _need_cuda(q_idx, reps, offsets, members, t, *[x for lv in levels for x in lv[:2]])
    B, d = q_idx.shape
    nl = len(levels)
    lib = _lib.load()
    rp = (ctypes.c_void_p * nl)(*[lv[0].data_ptr() for lv in levels])
    cp = (ctypes.c_void_p * nl)(*[lv[1].data_ptr() for lv in levels])
    ln = (ctypes.c_int32 * nl)(*[int(lv[0].shape[0]) for lv in levels])
    lk = (ctypes.c_int32 * nl)(*[int(lv[2]) for lv in levels])
    n_buckets = reps.shape[0]
    nbytes = lib.sa_bucket_tree_select_workspace(B, nl, ln, lk, n_buckets)
    ws = _workspace(nbytes, q_idx.device, ws)
    if out is None:
        idx = torch.empty((B, cap), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
    else:
        idx, n_sel = out
    buckets = torch.empty((B, top_b), dtype=torch.int32, device=q_idx.device) if return_buckets else None
    st = lib.sa_bucket_tree_select(_ptr(q_idx), _dtype(q_idx), B, d, nl, rp, cp, ln, lk, _ptr(reps), _ptr(offsets),
                                   _ptr(members), n_buckets, L, _ptr(t), top_b, n_sink, n_window, _ptr(idx),
                                   idx.stride(0), _ptr(n_sel), _ptr(buckets), _ptr(ws), nbytes, _stream(stream))
    _lib.check("sa_bucket_tree_select", st)
    return (idx, n_sel, buckets) if return_buckets else (idx, n_sel)


def sa_bucket_select_noalloc(q_idx, reps, offsets, members, L: int, top_b: int, n_sink: int = 0,
                             n_window: int = 0, cap: int = 8192, t=None, return_buckets: bool = False, out=None,
                             stream=None):
    """sa_bucket_select without a workspace (the library's static scratch array); out = (idx, n_sel[, buckets])
    preallocated by the caller, or None to have them allocated here."""
    _need_cuda(q_idx, reps, offsets, members, t)
    B, d = q_idx.shape
    nb = reps.shape[0]
    if out is None:
        idx = torch.empty((B, cap), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
        buckets = torch.empty((B, top_b), dtype=torch.int32, device=q_idx.device) if return_buckets else None
    else:
        idx, n_sel = out[0], out[1]
        buckets = out[2] if return_buckets else None
        cap = idx.stride(0)
    st = _lib.load().sa_bucket_select_noalloc(_ptr(q_idx), _dtype(q_idx), B, d, _ptr(reps), _ptr(offsets),
                                              _ptr(members), nb, L, _ptr(t), top_b, n_sink, n_window, _ptr(idx), cap,
                                              _ptr(n_sel), _ptr(buckets), _stream(stream))
    _lib.check("sa_bucket_select_noalloc", st)
    return (idx, n_sel, buckets) if return_buckets else (idx, n_sel)


def sa_hi_build(k_idx, sub_block: int, out=None, stream=None):
    """Mean index keys [ceil(L / sub_block), d] (bf16) of consecutive sub-blocks of the cache's index keys."""
    _need_cuda(k_idx)
    L, d = k_idx.shape
    n_sub = (L + sub_block - 1) // sub_block
    means = torch.empty((n_sub, d), dtype=torch.bfloat16, device=k_idx.device) if out is None else out
    if means.shape != (n_sub, d) or means.dtype != torch.bfloat16 or not means.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {(n_sub, d)}")
    st = _lib.load().sa_hi_build(_ptr(k_idx), _dtype(k_idx), _rows(k_idx), L, d, sub_block, _ptr(means),
                                 _stream(stream))
    _lib.check("sa_hi_build", st)
    return means


def sa_hi_select_workspace(L, B, sub_block, page_len, n_pages_keep, k_sparse) -> int:
    return int(_lib.load().sa_hi_select_workspace(L, B, sub_block, page_len, n_pages_keep, k_sparse))


def sa_hi_select(q_idx, w, k_idx, means, sub_block: int, page_len: int, n_pages_keep: int, k_sparse: int,
                 n_sink: int = 0, n_window: int = 0, t=None, idx_ld: Optional[int] = None, return_pages=False,
                 ws=None, out=None, stream=None):
    """(idx [B, idx_ld] ascending with -1 padding, n_sel [B][, pages [B, n_pages_keep]]) of the two-stage search."""
    _need_cuda(q_idx, w, k_idx, means, t)
    B, H, d = q_idx.shape
    L = k_idx.shape[0]
    if not means.is_contiguous() or means.shape != ((L + sub_block - 1) // sub_block, d):
        raise ValueError("means must be the contiguous output of sa_hi_build for this cache and sub_block")
    idx_ld = k_sparse if idx_ld is None else idx_ld
    lib = _lib.load()
    nbytes = lib.sa_hi_select_workspace(L, B, sub_block, page_len, n_pages_keep, k_sparse)
    ws = _workspace(nbytes, q_idx.device, ws)
    if out is None:
        idx = torch.empty((B, idx_ld), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
    else:
        idx, n_sel = out
    pages = torch.empty((B, n_pages_keep), dtype=torch.int32, device=q_idx.device) if return_pages else None
    st = lib.sa_hi_select(_ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_idx), _dtype(k_idx), _rows(k_idx), L, B, H, d,
                          _ptr(t), _ptr(means), sub_block, page_len, n_pages_keep, k_sparse, n_sink, n_window,
                          _ptr(idx), idx.stride(0), _ptr(n_sel), _ptr(pages), _ptr(ws), nbytes, _stream(stream))
    _lib.check("sa_hi_select", st)
    return (idx, n_sel, pages) if return_pages else (idx, n_sel)


def sa_qsa_pool(k_idx, block: int, out=None, stream=None):
    """Pooled index keys [ceil(L / block), d] (bf16): the mean of each micro-block's keys."""
    _need_cuda(k_idx)
    L, d = k_idx.shape
    n = (L + block - 1) // block
    pooled = torch.empty((n, d), dtype=torch.bfloat16, device=k_idx.device) if out is None else out
    if pooled.shape != (n, d) or pooled.dtype != torch.bfloat16 or not pooled.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 tensor of shape {(n, d)}")
    st = _lib.load().sa_qsa_pool(_ptr(k_idx), _dtype(k_idx), _rows(k_idx), L, d, block, _ptr(pooled),
                                 _stream(stream))
    _lib.check("sa_qsa_pool", st)
    return pooled


def sa_qsa_select(q_idx, w, pooled, L: int, block: int, k_blocks: int, t=None, idx_ld: Optional[int] = None,
                  ws=None, out=None, stream=None):
    """(idx [B, idx_ld] ascending with -1 padding, n_sel [B]): chosen micro-blocks expanded, then the tail."""
    _need_cuda(q_idx, w, pooled, t)
    B, H, d = q_idx.shape
    if not pooled.is_contiguous() or pooled.shape != ((L + block - 1) // block, d):
        raise ValueError("pooled must be the contiguous output of sa_qsa_pool for this cache and block")
    idx_ld = k_blocks * block + block - 1 if idx_ld is None else idx_ld
    lib = _lib.load()
    nbytes = lib.sa_qsa_select_workspace(L, B, H, d, block, k_blocks)
    ws = _workspace(nbytes, q_idx.device, ws)
    if out is None:
        idx = torch.empty((B, idx_ld), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B,), dtype=torch.int32, device=q_idx.device)
    else:
        idx, n_sel = out
    st = lib.sa_qsa_select(_ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(pooled), L, B, H, d, _ptr(t), block, k_blocks,
                           _ptr(idx), idx.stride(0), _ptr(n_sel), _ptr(ws), nbytes, _stream(stream))
    _lib.check("sa_qsa_select", st)
    return idx, n_sel


def sa_msa_select(q_idx, w, k_idx, G: int, block: int, k_blocks: int, t=None, idx_ld: Optional[int] = None,
                  ws=None, out=None, stream=None):
    """(idx [B * G, idx_ld] ascending with -1 padding, n_sel [B * G]): per (query, group) the chosen blocks whole,
    then the local block up to t."""
    _need_cuda(q_idx, w, k_idx, t)
    B, H, d = q_idx.shape
    L = k_idx.shape[0]
    idx_ld = k_blocks * block if idx_ld is None else idx_ld
    lib = _lib.load()
    nbytes = lib.sa_msa_select_workspace(L, B, G, block, k_blocks)
    ws = _workspace(nbytes, q_idx.device, ws)
    if out is None:
        idx = torch.empty((B * G, idx_ld), dtype=torch.int32, device=q_idx.device)
        n_sel = torch.empty((B * G,), dtype=torch.int32, device=q_idx.device)
    else:
        idx, n_sel = out
    st = lib.sa_msa_select(_ptr(q_idx), _dtype(q_idx), _ptr(w), _ptr(k_idx), _dtype(k_idx), _rows(k_idx), L, B, H,
                           d, G, _ptr(t), block, k_blocks, _ptr(idx), idx.stride(0), _ptr(n_sel), _ptr(ws), nbytes,
                           _stream(stream))
    _lib.check("sa_msa_select", st)
    return idx, n_sel


def sa_sparse_attn_workspace(B, H, d_qk, d_v, max_rows, dtype) -> int:
    return int(_lib.load().sa_sparse_attn_workspace(B, H, d_qk, d_v, max_rows, dtype))


def sa_sparse_attn(q, kv, idx, n_sel, n_sink: int, n_window: int, scale: float, t=None, v=None,
                   d_v: Optional[int] = None, return_lse: bool = False, ws=None, out=None, stream=None):
    """o [B, H, d_v] (and lse [B, H]) of softmax attention over sink U window U idx[b, :n_sel[b]] with logits
    scale * q . K (the caller's scale; idx and n_sel may both be None for sink and window only)."""
    _need_cuda(q, kv, idx, n_sel, t, v)
    B, H, d_qk = q.shape
    L = kv.shape[0]
    if d_v is None:
        d_v = v.shape[1] if v is not None else d_qk
    idx_ld = idx.stride(0) if idx is not None else 0
    lib = _lib.load()
    max_rows = n_sink + n_window + idx_ld
    nbytes = lib.sa_sparse_attn_workspace(B, H, d_qk, d_v, max_rows, _dtype(q))
    ws = _workspace(nbytes, q.device, ws)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if return_lse else None
    st = lib.sa_sparse_attn(_ptr(q), _ptr(kv), _ptr(v), _dtype(q), _rows(kv), _rows(v) if v is not None else 0, L, B,
                            H, d_qk, d_v, _ptr(t), _ptr(idx), idx_ld, _ptr(n_sel), n_sink, n_window, float(scale),
                            _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream))
    _lib.check("sa_sparse_attn", st)
    return (out, lse) if return_lse else out
