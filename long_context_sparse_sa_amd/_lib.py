"""ctypes loader for libsa.so (the C ABI declared in include/sa.h).

There is no fallback: if the HIP library is missing, importing the path raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SA_LIB_PATH selects another build of the same library (for instance one whose host code carries the address and
# undefined-behaviour sanitizers); the default is the in-tree build.
LIB_PATH = os.environ.get("SA_LIB_PATH") or os.path.join(HERE, "libsa.so")

SA_F32, SA_BF16, SA_E4M3 = 0, 1, 2
SA_TOPK_AUTO, SA_TOPK_SPLIT_L, SA_TOPK_PER_QUERY, SA_TOPK_RADIX, SA_TOPK_RADIX_LEVELS, SA_TOPK_STREAM = 0, 1, 2, 3, 4, 5
STATUS = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_DTYPE", 4: "SA_ERR_ALIGN",
          5: "SA_ERR_WORKSPACE", 6: "SA_ERR_UNSUPPORTED", 7: "SA_ERR_HIP"}

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
INT = ctypes.c_int
SZ = ctypes.c_size_t
F32 = ctypes.c_float

# name -> (restype, argtypes), in the order of include/sa.h
SIGNATURES = {
    "sa_status_string": (ctypes.c_char_p, [INT]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_version": (INT, []),
    "sa_index_score": (INT, [P, INT, P, P, INT, I64, I64, I32, I32, I32, P, I64, I64, P, I64, P]),
    "sa_select_topk_workspace": (SZ, [I64, I32, I32, I32, INT, INT, I32, INT]),
    "sa_select_topk": (INT, [P, INT, P, P, INT, I64, I64, I32, I32, I32, P, I32, I32, I32, P, I32, P, P, SZ, INT, P]),
    "sa_select_topk_scores_workspace": (SZ, [I64, I32]),
    "sa_select_topk_scores": (INT, [P, I64, I64, I32, P, I32, I32, I32, P, I32, P, P, SZ, P]),
    "sa_bucket_build_workspace": (SZ, [I64, I32]),
    "sa_bucket_build": (INT, [P, INT, I64, I64, I32, P, I32, P, P, P, P, SZ, P]),
    "sa_bucket_select_workspace": (SZ, [I32, I32, I32]),
    "sa_bucket_select": (INT, [P, INT, I32, I32, P, P, P, I32, I64, P, I32, I32, I32, P, I32, P, P, P, SZ, P]),
    "sa_bucket_tree_select_workspace": (SZ, [I32, I32, P, P, I32]),
    "sa_bucket_tree_select": (INT, [P, INT, I32, I32, I32, P, P, P, P, P, P, P, I32, I64, P, I32, I32, I32, P, I32, P,
                                    P, P, SZ, P]),
    "sa_bucket_select_noalloc_max_keys": (I64, []),
    "sa_bucket_select_noalloc": (INT, [P, INT, I32, I32, P, P, P, I32, I64, P, I32, I32, I32, P, I32, P, P, P]),
    "sa_hi_build": (INT, [P, INT, I64, I64, I32, I32, P, P]),
    "sa_hi_select_workspace": (SZ, [I64, I32, I32, I32, I32, I32]),
    "sa_hi_select": (INT, [P, INT, P, P, INT, I64, I64, I32, I32, I32, P, P, I32, I32, I32, I32, I32, I32, P, I32, P,
                           P, P, SZ, P]),
    "sa_qsa_pool": (INT, [P, INT, I64, I64, I32, I32, P, P]),
    "sa_qsa_select_workspace": (SZ, [I64, I32, I32, I32, I32, I32]),
    "sa_qsa_select": (INT, [P, INT, P, P, I64, I32, I32, I32, P, I32, I32, P, I32, P, P, SZ, P]),
    "sa_msa_select_workspace": (SZ, [I64, I32, I32, I32, I32]),
    "sa_msa_select": (INT, [P, INT, P, P, INT, I64, I64, I32, I32, I32, I32, P, I32, I32, P, I32, P, P, SZ, P]),
    "sa_sparse_attn_workspace": (SZ, [I32, I32, I32, I32, I64, INT]),
    "sa_sparse_attn": (INT, [P, P, P, INT, I64, I64, I64, I32, I32, I32, I32, P, P, I32, P, I32, I32, F32, P, P, P,
                             SZ, P]),
    "sa_set_stage_events": (None, [P, INT]),
    "sa_stage_events_used": (INT, []),
    "sa_set_stream_spin_limit": (None, [INT]),
}

_lib = None


class SAError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {msg}")
        self.status = status


def load():
    """Loads libsa.so once; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m long_context_sparse_sa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int):
    if status != 0:
        raise SAError(fn, status, load().sa_last_error().decode(errors="replace"))
