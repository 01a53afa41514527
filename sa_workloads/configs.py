"""Named workloads: the shapes, sizes and value distributions the sparse-attention path is measured and tested on.

The sizes follow the pages' settings where they give them: a 576-wide MLA latent row of 512 + 64 rope values
(AI LAB sheet 13.2 "K/V axis", historical section on DeepSeek V2; LongCat deep-dive, DSA baseline section), top-k
2048 for DSA-style selection (LongCat deep-dive, DSA baseline section), and the Flat bucket search with sink and
window positions (LSA eight-entry page, section 2). The pages run no public dataset on this path; every input here
is synthetic and seeded.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "dsa" (lightning indexer + top-k), "hi" (coarse-to-fine), "qsa" / "msa" (block
                              # indexers) or "bucket" (Flat search)
    L: int                    # cached positions
    B: int                    # queries
    # indexer
    H_I: int = 0              # indexer heads
    d_I: int = 0              # indexer dim
    idx_dtype: str = "bf16"   # storage dtype of q_idx and k_idx: f32 | bf16 | e4m3
    w_dist: str = "normal"    # distribution of the head weights w: normal | uniform
    k_sparse: int = 0
    # bucket directory
    n_buckets: int = 0
    top_b: int = 0
    tree_fan: int = 0         # Tree search: buckets per parent node (one parent level), parents kept per query
    tree_keep: int = 0
    key_noise: float = 0.3    # k = centre[assign] + key_noise * N(0, 1)
    # block-granular indexers: micro-block / block length, blocks kept, indexer head groups (MSA)
    block: int = 0
    k_blocks: int = 0
    groups: int = 1
    # coarse-to-fine index: sub-block mean keys, pages of sub-blocks, pages recalled per query
    sub_block: int = 0
    page_len: int = 0
    n_pages_keep: int = 0
    # selection budget
    n_sink: int = 0
    n_window: int = 0
    # main attention
    H: int = 128
    d_qk: int = 576
    d_v: int = 576
    attn_dtype: str = "bf16"  # f32 | bf16
    scale: Optional[float] = None
    # query positions: decode (all t = L-1) or a causal chunk of the last B positions
    causal_chunk: bool = False
    seed: int = 0

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d_qk)

    def t_positions(self):
        """Last visible position of each query."""
        if self.causal_chunk:
            return list(range(self.L - self.B, self.L))
        return [self.L - 1] * self.B

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Toy decode in fp32: 1 query, 4 indexer heads of width 32, latent of width 64 used as both K and V.
    "toy_decode_f32": Workload(
        name="toy_decode_f32", kind="dsa", L=1024, B=1, H_I=4, d_I=32, idx_dtype="f32", w_dist="uniform",
        k_sparse=64, n_sink=4, n_window=32, H=1, d_qk=64, d_v=64, attn_dtype="f32", scale=1.0 / 8.0),
    # DSA-style decode at 128K: 16 queries, 64 indexer heads x 128 (bf16), 128 query heads over a 576 bf16 latent.
    "dsa_decode_128k": Workload(
        name="dsa_decode_128k", kind="dsa", L=131072, B=16, H_I=64, d_I=128, idx_dtype="bf16", k_sparse=2048),
    # Prefill chunk: the last 32768 queries of a causal 128K sequence, same shapes as the 128K decode.
    "prefill_chunk_128k": Workload(
        name="prefill_chunk_128k", kind="dsa", L=131072, B=32768, H_I=64, d_I=128, idx_dtype="bf16",
        k_sparse=2048, causal_chunk=True),
    # Flat bucket search at 1M: 16384 centres, keys = centre + 0.3 N(0,1), top 32 buckets + sink 4 + window 128.
    "lsa_flat_1m": Workload(
        name="lsa_flat_1m", kind="bucket", L=1 << 20, B=8, d_I=128, idx_dtype="bf16", n_buckets=16384, top_b=32,
        n_sink=4, n_window=128),
    # The Tree search over the same directory: one parent level of 128 nodes over 128 buckets each; each query keeps
    # its 8 best parents and chooses its top 32 buckets among their 1024 children (fan-out and beam are readings:
    # the pages give neither).
    "lsa_tree_1m": Workload(
        name="lsa_tree_1m", kind="bucket", L=1 << 20, B=8, d_I=128, idx_dtype="bf16", n_buckets=16384, top_b=32,
        n_sink=4, n_window=128, tree_fan=128, tree_keep=8),
    # A prefill chunk of 2048 queries at the end of a causal 1M sequence (the query length of the LongCat
    # deep-dive's HI-versus-flat table), selected by the coarse-to-fine index: sub-blocks of 8, pages of 128, the
    # best 1024 pages recalled per query (the settings of that section), then the top 2048 inside them.
    "hi_prefill_1m": Workload(
        name="hi_prefill_1m", kind="hi", L=1 << 20, B=2048, H_I=64, d_I=128, idx_dtype="bf16", k_sparse=2048,
        sub_block=8, page_len=128, n_pages_keep=1024, causal_chunk=True),
    # The same chunk selected by the flat indexer (every visible position scored): the table's other column.
    "flat_prefill_1m": Workload(
        name="flat_prefill_1m", kind="dsa", L=1 << 20, B=2048, H_I=64, d_I=128, idx_dtype="bf16", k_sparse=2048,
        causal_chunk=True),
    # The 128K decode with QSA micro-blocks: index keys pooled over 4 positions, 512 micro-blocks (the release
    # budget of 2048 tokens) plus the unfinished micro-block's tail ("long-context attention" lecture, QSA section).
    "qsa_decode_128k": Workload(
        name="qsa_decode_128k", kind="qsa", L=131072, B=16, H_I=64, d_I=128, idx_dtype="bf16", block=4,
        k_blocks=512),
    # The 128K decode with MSA blocks: two groups of 32 indexer heads (each group's 64 query heads share its
    # selection), blocks of 128, 16 blocks per group including the local block (the lecture's MSA settings).
    "msa_decode_128k": Workload(
        name="msa_decode_128k", kind="msa", L=131072, B=16, H_I=64, d_I=128, idx_dtype="bf16", block=128,
        k_blocks=16, groups=2),
    # 10M-token decode with fp8 E4M3 index keys and queries, fp32 accumulation; 4 queries.
    "decode_10m_fp8": Workload(
        name="decode_10m_fp8", kind="dsa", L=10_000_000, B=4, H_I=64, d_I=128, idx_dtype="e4m3", k_sparse=2048,
        n_sink=4, n_window=128),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.with_(**overrides) if overrides else w
