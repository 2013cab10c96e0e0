"""ctypes loader for libmsa.so: declares the C ABI of include/msa.h.  Fails loudly when the
library has not been built -- there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

c_i32, c_i64, c_f32, c_size, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

MSA_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED", 3: "MSA_ERR_WORKSPACE_TOO_SMALL",
              4: "MSA_ERR_HIP"}

# Every symbol include/msa.h declares.
EXPORTS = ("msa_index_score", "msa_index_topk", "msa_index_topk_workspace_size", "msa_topk_blocks", "msa_build_sparse_page_table",
           "msa_topk_page_table", "msa_topk_attn_decode", "msa_topk_attn_decode_noalloc", "msa_sparse_attn_decode",
           "msa_sparse_attn_decode_workspace_size", "msa_sparse_attn_prefill",
           "msa_sparse_attn_prefill_workspace_size", "msa_lse_merge", "msa_status_string", "msa_last_error",
           "msa_version")


class MsaBatch(ctypes.Structure):
    _fields_ = [("num_requests", c_i32), ("num_queries", c_i32), ("max_blocks", c_i32),
                ("max_q_per_request", c_i32), ("block_table", c_vp), ("ctx_len", c_vp), ("cu_q", c_vp),
                ("q_pos", c_vp)]


class MsaCache(ctypes.Structure):
    _fields_ = [("data", c_vp), ("num_pages", c_i32), ("block_size", c_i32), ("num_heads", c_i32),
                ("head_dim", c_i32), ("page_stride", c_i64)]


_SIGS = {
    "msa_index_score": (c_i32, [ctypes.POINTER(MsaBatch), c_vp, MsaCache, c_vp, c_vp]),
    "msa_topk_blocks": (c_i32, [ctypes.POINTER(MsaBatch), c_i32, c_vp, c_i32, c_vp, c_vp, c_vp]),
    "msa_index_topk": (c_i32, [ctypes.POINTER(MsaBatch), c_vp, MsaCache, c_i32, c_vp, c_vp, c_vp, c_size, c_vp]),
    "msa_index_topk_workspace_size": (c_size, [ctypes.POINTER(MsaBatch), c_i32, c_i32]),
    "msa_build_sparse_page_table": (c_i32, [ctypes.POINTER(MsaBatch), MsaCache, c_vp, c_vp, c_i32, c_vp, c_vp,
                                            c_vp]),
    "msa_topk_page_table": (c_i32, [ctypes.POINTER(MsaBatch), MsaCache, c_vp, c_i32, c_vp, c_vp, c_vp, c_vp,
                                    c_vp]),
    "msa_topk_attn_decode": (c_i32, [ctypes.POINTER(MsaBatch), c_vp, c_i32, MsaCache, MsaCache, c_i32, c_vp, c_f32,
                                     c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "msa_topk_attn_decode_noalloc": (c_i32, [ctypes.POINTER(MsaBatch), c_vp, c_i32, MsaCache, MsaCache, c_i32, c_vp,
                                             c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "msa_sparse_attn_decode": (c_i32, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_f32,
                                       c_vp, c_vp, c_vp, c_size, c_vp]),
    "msa_sparse_attn_decode_workspace_size": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "msa_sparse_attn_prefill": (c_i32, [ctypes.POINTER(MsaBatch), c_i32, c_vp, MsaCache, MsaCache, c_vp, c_vp, c_i32,
                                        c_f32, c_i32, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "msa_sparse_attn_prefill_workspace_size": (c_size, [ctypes.POINTER(MsaBatch), c_i32, c_i32]),
    "msa_lse_merge": (c_i32, [c_i64, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "msa_status_string": (ctypes.c_char_p, [c_i32]),
    "msa_last_error": (ctypes.c_char_p, []),
    "msa_version": (c_i32, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libmsa.so (once) and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m block_sparse_long_msa_amd.build` "
                           "(or __graft_entry__.build()) first; there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MSAError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with {MSA_STATUS.get(status, status)}: {message}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise MSAError(fn, status, load().msa_last_error().decode())
