"""Builds libsa.so (the C ABI in include/sa.h) for gfx950 with hipcc, in-tree next to this file.

Usage: python -m long_context_sparse_sa_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libsa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["sa_api.cpp", "k_index.hip", "k_select.hip", "k_radix.hip", "k_bucket.hip", "k_attn.hip", "k_hi.hip",
           "k_blocks.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source extra flags. The attention and indexer kernels keep their MFMA accumulators in VGPRs: their
# epilogues (online-softmax rescale; ReLU and head weights) work on them with VALU instructions, and the default
# AGPR form copies them between the two register files on every tile.
EXTRA = {"k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "k_index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_hi.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), *lang, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    args = ap.parse_args()
    try:
        build(args.jobs, verbose=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
