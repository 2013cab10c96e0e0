"""MiniMax Sparse Attention (MSA) hot path for AMD MI355X: Python binding of libmsa.so.

Each function has the name of the C entry point it calls (see include/msa.h) and only
marshals arguments: torch tensors become device pointers, the current HIP stream is passed
along, and a non-OK status raises MSAError.  All computation happens in the HIP kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from ._lib import EXPORTS, MsaBatch, MsaCache, MSAError, check, load  # noqa: F401

__all__ = ["Batch", "HostResident", "MSAError", "msa_index_score", "msa_index_topk", "msa_index_topk_workspace_size",
           "msa_topk_blocks", "msa_build_sparse_page_table", "msa_topk_page_table", "msa_topk_attn_decode",
           "msa_topk_attn_decode_noalloc", "msa_sparse_attn_decode", "msa_sparse_attn_decode_workspace_size", "msa_sparse_attn_prefill",
           "msa_sparse_attn_prefill_workspace_size", "msa_lse_merge", "msa_version", "load"]


_hip = None


def _host_device_pointer(host_ptr: int) -> int:
    """Device address of pinned host memory (hipHostGetDevicePointer)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipHostGetDevicePointer.restype = ctypes.c_int
        _hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    dev = ctypes.c_void_p()
    err = _hip.hipHostGetDevicePointer(ctypes.byref(dev), ctypes.c_void_p(host_ptr), 0)
    if err != 0 or not dev.value:
        raise RuntimeError(f"hipHostGetDevicePointer failed ({err}): the tensor is not device-accessible pinned memory")
    return dev.value


class HostResident:
    """A pinned host tensor that the kernels read in place over the host link, e.g. K/V caches moved
    out of HBM while the key-index cache stays resident: each decode step then fetches only the
    selected blocks (the decoupled index/value offload that the Chinese page, section "遗留问题",
    leaves as future work).  Wrap a tensor from ``t.pin_memory()`` or ``torch.empty(..., pin_memory=True)``;
    it can be passed wherever a cache or K/V base tensor is expected."""

    def __init__(self, t: torch.Tensor):
        if t.is_cuda or not t.is_pinned():
            raise ValueError("HostResident needs a pinned CPU tensor")
        if not t.is_contiguous():
            raise ValueError("HostResident needs a contiguous tensor")
        self.tensor = t
        self.shape, self.dtype = t.shape, t.dtype
        self.device_ptr = _host_device_pointer(t.data_ptr())

    def dim(self) -> int:
        return self.tensor.dim()


def _ptr(t, dtype, name: str, allow_none: bool = False) -> Optional[int]:
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if isinstance(t, HostResident):
        if t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
        return t.device_ptr
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _base(t, name: str) -> int:
    """Base address of a strided view (the call's strides say how it is walked)."""
    if isinstance(t, HostResident):
        return _ptr(t, torch.bfloat16, name)
    if not t.is_cuda or t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be a bf16 GPU tensor")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _cache(t, name: str) -> MsaCache:
    """A paged cache [pages, block, heads, dim] whose token rows are contiguous.  The pages may be spaced
    apart (a view such as pool[:, 0] of a [pages, 2, block, heads, dim] pool): the page dimension's
    stride becomes the cache's page_stride."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [pages, block, heads, dim]")
    P, BS, H, D = t.shape
    if isinstance(t, HostResident):
        return MsaCache(_ptr(t, torch.bfloat16, name), P, BS, H, D, 0)
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be {torch.bfloat16}, got {t.dtype}")
    s = t.stride()
    if s[3] != 1 or s[2] != D or s[1] != H * D:
        raise ValueError(f"{name}: each page's [block, heads, dim] elements must be contiguous (only the page "
                         f"dimension may be strided), got strides {tuple(s)}")
    page_stride = 0 if (P == 1 or s[0] == BS * H * D) else s[0]
    return MsaCache(t.data_ptr(), P, BS, H, D, page_stride)


class Batch:
    """Requests and query rows (all int32 GPU tensors): block_table [B, max_blocks], ctx_len [B],
    cu_q [B+1], q_pos [Nq].  ``max_q_per_request`` is the host-side bound on queries per request."""

    def __init__(self, block_table, ctx_len, cu_q, q_pos, max_q_per_request: int):
        self.block_table, self.ctx_len, self.cu_q, self.q_pos = block_table, ctx_len, cu_q, q_pos
        self.max_q_per_request = int(max_q_per_request)
        B = ctx_len.shape[0]
        if block_table.dim() != 2 or block_table.shape[0] != B or cu_q.shape[0] != B + 1:
            raise ValueError("block_table must be [B, max_blocks] and cu_q [B+1]")
        self._c = MsaBatch(B, q_pos.shape[0], block_table.shape[1], self.max_q_per_request,
                           _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_len, torch.int32, "ctx_len"),
                           _ptr(cu_q, torch.int32, "cu_q"), _ptr(q_pos, torch.int32, "q_pos"))

    @property
    def num_requests(self) -> int:
        return self._c.num_requests

    @property
    def num_queries(self) -> int:
        return self._c.num_queries

    @property
    def max_blocks(self) -> int:
        return self._c.max_blocks

    def ref(self):
        return ctypes.byref(self._c)


def msa_index_score(batch: Batch, q_idx, k_idx, scores, stream=None) -> None:
    check("msa_index_score", load().msa_index_score(batch.ref(), _ptr(q_idx, torch.bfloat16, "q_idx"),
                                                     _cache(k_idx, "k_idx"), _ptr(scores, torch.float32, "scores"),
                                                     _stream(stream)))


def msa_index_topk_workspace_size(batch: Batch, num_kv_heads: int, k: int) -> int:
    return int(load().msa_index_topk_workspace_size(batch.ref(), num_kv_heads, k))


def msa_index_topk(batch: Batch, q_idx, k_idx, k: int, sel, cnt, workspace=None, stream=None) -> None:
    ws = _ptr(workspace, torch.uint8, "workspace", True)
    check("msa_index_topk", load().msa_index_topk(batch.ref(), _ptr(q_idx, torch.bfloat16, "q_idx"),
                                                   _cache(k_idx, "k_idx"), k, _ptr(sel, torch.int32, "sel"),
                                                   _ptr(cnt, torch.int32, "cnt"), ws,
                                                   0 if workspace is None else workspace.numel(), _stream(stream)))


def msa_topk_blocks(batch: Batch, num_kv_heads: int, scores, k: int, sel, cnt, stream=None) -> None:
    check("msa_topk_blocks", load().msa_topk_blocks(batch.ref(), num_kv_heads, _ptr(scores, torch.float32, "scores"),
                                                     k, _ptr(sel, torch.int32, "sel"), _ptr(cnt, torch.int32, "cnt"),
                                                     _stream(stream)))


def msa_build_sparse_page_table(batch: Batch, kv_layout, sel, cnt, k: int, page_table, row_len, stream=None) -> None:
    """kv_layout: the K (or V) cache tensor; only its shape and page stride are used."""
    check("msa_build_sparse_page_table",
          load().msa_build_sparse_page_table(batch.ref(), _cache(kv_layout, "kv_layout"), _ptr(sel, torch.int32, "sel"),
                                             _ptr(cnt, torch.int32, "cnt"), k,
                                             _ptr(page_table, torch.int32, "page_table"),
                                             _ptr(row_len, torch.int32, "row_len"), _stream(stream)))


def msa_topk_page_table(batch: Batch, kv_layout, scores, k: int, sel, cnt, page_table, row_len, stream=None) -> None:
    """kv_layout: the K (or V) cache tensor; only its shape and page stride are used."""
    check("msa_topk_page_table",
          load().msa_topk_page_table(batch.ref(), _cache(kv_layout, "kv_layout"), _ptr(scores, torch.float32, "scores"),
                                     k,
                                     _ptr(sel, torch.int32, "sel"), _ptr(cnt, torch.int32, "cnt"),
                                     _ptr(page_table, torch.int32, "page_table"),
                                     _ptr(row_len, torch.int32, "row_len"), _stream(stream)))


def msa_topk_attn_decode(batch: Batch, scores, k: int, k_cache, v_cache, G: int, q, sm_scale: float, sel, cnt,
                         page_table, row_len, out, lse, workspace, stream=None) -> None:
    check("msa_topk_attn_decode",
          load().msa_topk_attn_decode(batch.ref(), _ptr(scores, torch.float32, "scores"), k, _cache(k_cache, "k_cache"),
                                      _cache(v_cache, "v_cache"), G, _ptr(q, torch.bfloat16, "q"), sm_scale,
                                      _ptr(sel, torch.int32, "sel"), _ptr(cnt, torch.int32, "cnt"),
                                      _ptr(page_table, torch.int32, "page_table"),
                                      _ptr(row_len, torch.int32, "row_len"), _ptr(out, torch.bfloat16, "out"),
                                      _ptr(lse, torch.float32, "lse", True),
                                      _ptr(workspace, torch.uint8, "workspace", True),
                                      0 if workspace is None else workspace.numel(), _stream(stream)))


def msa_topk_attn_decode_noalloc(batch: Batch, scores, k: int, k_cache, v_cache, G: int, q, sm_scale: float, sel,
                                 cnt, page_table, row_len, out, lse, stream=None) -> None:
    check("msa_topk_attn_decode_noalloc",
          load().msa_topk_attn_decode_noalloc(batch.ref(), _ptr(scores, torch.float32, "scores"), k,
                                              _cache(k_cache, "k_cache"), _cache(v_cache, "v_cache"), G,
                                              _ptr(q, torch.bfloat16, "q"), sm_scale, _ptr(sel, torch.int32, "sel"),
                                              _ptr(cnt, torch.int32, "cnt"),
                                              _ptr(page_table, torch.int32, "page_table"),
                                              _ptr(row_len, torch.int32, "row_len"), _ptr(out, torch.bfloat16, "out"),
                                              _ptr(lse, torch.float32, "lse", True), _stream(stream)))


def msa_sparse_attn_decode_workspace_size(rows: int, G: int, D: int, k: int) -> int:
    return int(load().msa_sparse_attn_decode_workspace_size(rows, G, D, k))


def msa_sparse_attn_decode(rows: int, G: int, D: int, q, k_base, v_base, page_stride: int, token_stride: int,
                           page_table, k: int, row_len, sm_scale: float, out, lse, workspace, stream=None) -> None:
    check("msa_sparse_attn_decode",
          load().msa_sparse_attn_decode(rows, G, D, _ptr(q, torch.bfloat16, "q"), _base(k_base, "k_base"),
                                        _base(v_base, "v_base"), page_stride, token_stride,
                                        _ptr(page_table, torch.int32, "page_table"), k,
                                        _ptr(row_len, torch.int32, "row_len"), sm_scale,
                                        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse", True),
                                        _ptr(workspace, torch.uint8, "workspace", True),
                                        0 if workspace is None else workspace.numel(), _stream(stream)))


def msa_sparse_attn_prefill_workspace_size(batch: Batch, num_kv_heads: int, k: int) -> int:
    return int(load().msa_sparse_attn_prefill_workspace_size(batch.ref(), num_kv_heads, k))


def msa_sparse_attn_prefill(batch: Batch, G: int, q, k_cache, v_cache, sel, cnt, k: int, sm_scale: float, part_o,
                            part_lse, workspace, stream=None, tile_min_rows: int = 0, slot_of=None) -> None:
    check("msa_sparse_attn_prefill",
          load().msa_sparse_attn_prefill(batch.ref(), G, _ptr(q, torch.bfloat16, "q"), _cache(k_cache, "k_cache"),
                                         _cache(v_cache, "v_cache"), _ptr(sel, torch.int32, "sel"),
                                         _ptr(cnt, torch.int32, "cnt"), k, sm_scale, tile_min_rows,
                                         _ptr(part_o, torch.bfloat16, "part_o"),
                                         _ptr(part_lse, torch.float32, "part_lse"),
                                         _ptr(slot_of, torch.int32, "slot_of", True),
                                         _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
                                         _stream(stream)))


def msa_lse_merge(rows: int, parts: int, G: int, D: int, part_o, part_lse, out, lse_out, stream=None) -> None:
    check("msa_lse_merge", load().msa_lse_merge(rows, parts, G, D, _ptr(part_o, torch.bfloat16, "part_o"),
                                                 _ptr(part_lse, torch.float32, "part_lse"),
                                                 _ptr(out, torch.bfloat16, "out"),
                                                 _ptr(lse_out, torch.float32, "lse_out", True), _stream(stream)))


def msa_version() -> int:
    return int(load().msa_version())
