"""Byte and flop accounting for the sparse-attention path (what a kernel must move or compute, not what it does).

The byte formulas follow the pages' own accounting: stored bytes count every cached row, read bytes count only the
selected rows, and an index directory is counted separately (LSA eight-entry page, section 3); a full K/V cache
takes 2 x layers x H_kv x d x S x bytes, an MLA latent cache layers x (d_c + d_rope) x S x bytes with no factor 2
(AI LAB sheet 13.2, section 04).
"""
from __future__ import annotations

ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}

# MI355X published peaks used as roofline denominators.
PEAK_HBM_GBPS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "e4m3": 5000.0, "f32_vector": 157.3, "f64_vector": 78.6}


def stored_bytes(n_rows: int, numbers_per_row: int, bytes_per_number: int) -> int:
    return n_rows * numbers_per_row * bytes_per_number


def read_bytes(n_selected: int, numbers_per_row: int, bytes_per_number: int) -> int:
    return n_selected * numbers_per_row * bytes_per_number


def directory_bytes(n_reps: int, rep_dim: int, bytes_per_number: int, n_positions: int, position_bytes: int) -> int:
    return n_reps * rep_dim * bytes_per_number + n_positions * position_bytes


def kv_cache_bytes_mha(layers: int, H_kv: int, d: int, S: int, bytes_per_number: int) -> int:
    return 2 * layers * H_kv * d * S * bytes_per_number


def kv_cache_bytes_mla(layers: int, d_c: int, d_rope: int, S: int, bytes_per_number: int) -> int:
    return layers * (d_c + d_rope) * S * bytes_per_number


# ---- per-kernel algorithmic work ---------------------------------------------------------------------------------


def attn_bytes(n_rows_total: int, B: int, H: int, d_qk: int, d_v: int, row_width: int, dtype: str) -> int:
    """Gathered rows + queries + outputs of one sparse-attention launch."""
    e = ELEM_BYTES[dtype]
    return n_rows_total * row_width * e + B * H * d_qk * e + B * H * d_v * e


def attn_flops(n_rows_total: int, H: int, d_qk: int, d_v: int) -> int:
    """q.K and P.V multiply-adds (2 flops each) for every (row, head) pair."""
    return 2 * n_rows_total * H * (d_qk + d_v)


def indexer_bytes(n_keys: int, B: int, H_I: int, d_I: int, dtype: str) -> int:
    e = ELEM_BYTES[dtype]
    return n_keys * d_I * e + B * H_I * d_I * e + B * H_I * 4


def indexer_flops(n_pairs: int, H_I: int, d_I: int) -> int:
    """Dot products (2 flops per multiply-add) for every scored (query, key) pair over all heads."""
    return 2 * n_pairs * H_I * d_I
