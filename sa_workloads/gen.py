"""Seeded input generation. Only random draws and storage casts live here; no step of the method does.

Every tensor is drawn from its own torch generator, seeded from (seed, tag), so each tensor is reproducible on
its own. Values are drawn in fp32 and then cast (round-to-nearest-even) to the storage dtype; the stored bytes are
what both the oracle and the HIP path consume.

Recipes (synthetic stand-ins for the pages' workloads):
  q_idx, k_idx, q, latent kv ~ N(0, 1); w ~ N(0, 1), or U(0, 1) for the fp32 toy.
  bucket workloads: centres ~ N(0, 1) [n_buckets, d], assign ~ U{0..n_buckets-1},
  k = centre[assign] + key_noise * N(0, 1).
"""
from __future__ import annotations

import zlib
from typing import Dict, Iterable

import torch

STORAGE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}
RAW_VIEW = {"f32": torch.int32, "bf16": torch.int16, "e4m3": torch.uint8}

_CHUNK = 1 << 26  # elements drawn per call for large tensors


def _generator(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 0x9E3779B1 + zlib.crc32(tag.encode())) & 0x7FFFFFFFFFFFFFFF)
    return g


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(STORAGE[dtype])


def normal(shape, seed: int, tag: str, device="cpu", dtype: str = "f32", scale: float = 1.0) -> torch.Tensor:
    """N(0, scale^2) draws cast to the storage dtype; drawn in chunks so huge tensors never need an fp32 copy."""
    g = _generator(seed, tag, device)
    out = torch.empty(shape, dtype=STORAGE[dtype], device=device)
    flat = out.view(-1)
    for lo in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - lo)
        x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[lo:lo + n] = x.to(STORAGE[dtype])
    return out


def uniform(shape, seed: int, tag: str, device="cpu") -> torch.Tensor:
    g = _generator(seed, tag, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def randint(high: int, shape, seed: int, tag: str, device="cpu") -> torch.Tensor:
    g = _generator(seed, tag, device)
    return torch.randint(0, high, shape, generator=g, device=device, dtype=torch.int64).to(torch.int32)


def bucket_keys(wl, seed: int, device="cpu"):
    """Clustered index keys: each position joins a uniform-random centre and adds key_noise * N(0, 1)."""
    centres = normal((wl.n_buckets, wl.d_I), seed, "centres", device)
    assign = randint(wl.n_buckets, (wl.L,), seed, "assign", device)
    k = torch.empty((wl.L, wl.d_I), dtype=STORAGE[wl.idx_dtype], device=device)
    g = _generator(seed, "key_noise", device)
    rows = max(1, _CHUNK // wl.d_I)
    for lo in range(0, wl.L, rows):
        hi = min(wl.L, lo + rows)
        noise = torch.randn((hi - lo, wl.d_I), generator=g, device=device, dtype=torch.float32)
        k[lo:hi] = (centres[assign[lo:hi].long()] + wl.key_noise * noise).to(STORAGE[wl.idx_dtype])
    return centres, assign, k


def make_inputs(wl, device="cpu", seed: int = None, parts: Iterable[str] = ("index", "attn")) -> Dict[str, torch.Tensor]:
    """All inputs of one workload in their storage dtypes on `device`.

    parts: "index" -> indexer (or bucket) inputs; "attn" -> query heads and the latent cache.
    """
    seed = wl.seed if seed is None else seed
    parts = set(parts)
    out: Dict[str, torch.Tensor] = {
        "t": torch.tensor(wl.t_positions(), dtype=torch.int32, device=device),
    }
    if "index" in parts:
        if wl.kind in ("dsa", "hi", "qsa", "msa"):
            out["q_idx"] = normal((wl.B, wl.H_I, wl.d_I), seed, "q_idx", device, wl.idx_dtype)
            if wl.w_dist == "uniform":
                out["w"] = uniform((wl.B, wl.H_I), seed, "w", device)
            else:
                out["w"] = normal((wl.B, wl.H_I), seed, "w", device)
            out["k_idx"] = normal((wl.L, wl.d_I), seed, "k_idx", device, wl.idx_dtype)
        elif wl.kind == "bucket":
            _, assign, k = bucket_keys(wl, seed, device)
            out["assign"] = assign
            out["k_idx"] = k
            out["q_idx"] = normal((wl.B, wl.d_I), seed, "q_idx", device, wl.idx_dtype)
        else:
            raise ValueError(wl.kind)
    if "attn" in parts:
        width = max(wl.d_qk, wl.d_v)
        out["q"] = normal((wl.B, wl.H, wl.d_qk), seed, "q", device, wl.attn_dtype)
        out["kv"] = normal((wl.L, width), seed, "kv", device, wl.attn_dtype)
    return out


def raw_bytes(x: torch.Tensor, dtype: str):
    """The stored bit patterns of a storage tensor as a numpy array (uint32 / uint16 / uint8)."""
    import numpy as np
    v = x.detach().cpu().contiguous().view(RAW_VIEW[dtype]).numpy()
    return v.view({"f32": np.uint32, "bf16": np.uint16, "e4m3": np.uint8}[dtype])
