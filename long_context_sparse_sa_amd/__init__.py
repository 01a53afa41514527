"""Retrieval-sparse attention for long contexts on AMD MI355X (gfx950).

The hot path -- indexer scoring, exact top-k with sink/window budget (or Flat bucket search), and sparse
attention over the gathered latent rows -- runs in hand-written HIP kernels behind the C ABI of include/sa.h.
This package is the thin Python binding of that library.
"""
from ._lib import (SA_BF16, SA_E4M3, SA_F32, SA_TOPK_AUTO, SA_TOPK_PER_QUERY, SA_TOPK_RADIX, SA_TOPK_RADIX_LEVELS,
                   SA_TOPK_SPLIT_L, SA_TOPK_STREAM, SAError, load)
from .api import (sa_bucket_build, sa_bucket_select, sa_bucket_select_noalloc, sa_bucket_tree_select, sa_hi_build, sa_hi_select,
                  sa_hi_select_workspace, sa_index_score, sa_msa_select, sa_qsa_pool, sa_qsa_select, sa_select_topk, sa_select_topk_scores,
                  sa_select_topk_workspace, sa_sparse_attn, sa_sparse_attn_workspace)

__all__ = ["SA_F32", "SA_BF16", "SA_E4M3", "SA_TOPK_AUTO", "SA_TOPK_SPLIT_L", "SA_TOPK_PER_QUERY", "SA_TOPK_RADIX", "SA_TOPK_RADIX_LEVELS", "SA_TOPK_STREAM", "SAError", "load",
           "sa_index_score", "sa_select_topk", "sa_select_topk_scores", "sa_select_topk_workspace", "sa_bucket_build", "sa_bucket_select", "sa_bucket_select_noalloc", "sa_bucket_tree_select",
           "sa_hi_build", "sa_hi_select", "sa_hi_select_workspace",
           "sa_qsa_pool", "sa_qsa_select", "sa_msa_select", "sa_sparse_attn", "sa_sparse_attn_workspace"]
