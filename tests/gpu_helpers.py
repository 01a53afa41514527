"""Shared helpers of the GPU parity tests: move stored tensors to the oracle (fp64) and compare selections."""
from __future__ import annotations

import numpy as np
import torch

from oracle import sa_oracle as O

DT_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float8_e4m3fn: "e4m3"}
RAW = {torch.float32: (torch.int32, np.uint32), torch.bfloat16: (torch.int16, np.uint16),
       torch.float8_e4m3fn: (torch.uint8, np.uint8)}


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a stored tensor, decoded by the oracle from its bit patterns."""
    tv, nv = RAW[x.dtype]
    raw = x.detach().cpu().contiguous().view(tv).numpy().view(nv)
    return O.decode(raw, DT_NAME[x.dtype])


def band_compare(gpu_sel, ora_sel, cand, score32, k, rel=1e-5):
    """Selected sets agree outside the band of candidates whose fp32 score lies within `rel` of the k-th score."""
    gpu_sel = np.asarray(gpu_sel, dtype=np.int64)
    ora_sel = np.asarray(ora_sel, dtype=np.int64)
    assert gpu_sel.size == ora_sel.size, (gpu_sel.size, ora_sel.size)
    assert np.all(np.diff(gpu_sel) > 0), "idx must be strictly ascending"
    assert np.all(np.isin(gpu_sel, cand)), "idx holds a non-candidate position"
    if ora_sel.size == cand.size:
        np.testing.assert_array_equal(gpu_sel, ora_sel)
        return 0
    kth = O.kth_score(score32, cand, k)
    s = np.asarray(score32, dtype=np.float64)
    band = cand[np.abs(s - kth) <= rel * max(abs(kth), 1e-30)]
    g = np.setdiff1d(gpu_sel, band)
    o = np.setdiff1d(ora_sel, band)
    np.testing.assert_array_equal(g, o)
    return band.size


def selected(idx_row: torch.Tensor, n: int) -> np.ndarray:
    row = idx_row.cpu().numpy()
    assert np.all(row[n:] == -1), "padding must be -1"
    return row[:n].astype(np.int64)
