"""One MSA layer invocation as a chain of C-ABI calls with preallocated buffers.

MSADecode: index scores -> top-k + sparse page table + decode attention (split over pages,
           merged in the library), by default in one call after the scores.
MSAPrefill: index scores + top-k (one fused call by default) -> KV-block-major attention (partials)
           -> LSE merge.
MSAPrefillQueryMajor: the query-major baseline the KV-block-major mapping is measured against:
           index scores -> top-k + page table -> every (query token, KV head) row attends to its own
           k blocks with the paged decode kernel (no partials, no merge, K/V re-read per row).

Buffers are allocated once with torch (device memory only); every step runs in libmsa.so.
"""
from __future__ import annotations

import torch

from . import (Batch, msa_build_sparse_page_table, msa_index_score, msa_index_topk, msa_index_topk_workspace_size,
               msa_lse_merge, msa_sparse_attn_decode, msa_sparse_attn_decode_workspace_size,
               msa_sparse_attn_prefill, msa_sparse_attn_prefill_workspace_size, msa_topk_attn_decode,
               msa_topk_blocks, msa_topk_page_table)


class MSADecode:
    """``select_mode`` picks how the blocks are selected and attended after the scores:
    "attend" (default): msa_topk_attn_decode, top-k + page table + attention in one launch;
    "page_table": msa_topk_page_table, then msa_sparse_attn_decode;
    "separate": msa_topk_blocks, msa_build_sparse_page_table, then msa_sparse_attn_decode.
    All three give bit-identical results and fill the same buffers."""

    MODES = ("attend", "page_table", "separate")

    def __init__(self, batch: Batch, Hkv: int, G: int, D: int, k: int, num_pages: int, device="cuda",
                 select_mode: str = "attend"):
        if select_mode not in self.MODES:
            raise ValueError(f"select_mode must be one of {self.MODES}, got {select_mode!r}")
        Nq, mb = batch.num_queries, batch.max_blocks
        self.batch, self.Hkv, self.G, self.D, self.k, self.num_pages = batch, Hkv, G, D, k, num_pages
        self.select_mode = select_mode
        self.rows = Nq * Hkv
        self.scores = torch.empty((Nq, Hkv, mb), dtype=torch.float32, device=device)
        self.sel = torch.empty((Nq, Hkv, k), dtype=torch.int32, device=device)
        self.cnt = torch.empty((Nq, Hkv), dtype=torch.int32, device=device)
        self.page_table = torch.empty((self.rows, k), dtype=torch.int32, device=device)
        self.row_len = torch.empty((self.rows,), dtype=torch.int32, device=device)
        self.out = torch.empty((Nq, Hkv * G, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((Nq, Hkv * G), dtype=torch.float32, device=device)
        # zeroed once: the split merge's row arrival counters at its end start at zero
        self.ws = torch.zeros((msa_sparse_attn_decode_workspace_size(self.rows, G, D, k),), dtype=torch.uint8,
                              device=device)

    def score(self, q_idx, kidx, stream=None):
        msa_index_score(self.batch, q_idx, kidx, self.scores, stream)

    def select(self, kcache, stream=None):
        """Top-k and page table only (the "page_table" and "separate" modes); the page ids follow the K
        cache's layout (its page stride)."""
        if self.select_mode == "separate":
            msa_topk_blocks(self.batch, self.Hkv, self.scores, self.k, self.sel, self.cnt, stream)
            msa_build_sparse_page_table(self.batch, kcache, self.sel, self.cnt, self.k, self.page_table, self.row_len,
                                        stream)
        else:
            msa_topk_page_table(self.batch, kcache, self.scores, self.k, self.sel, self.cnt, self.page_table,
                                self.row_len, stream)

    def attend(self, q, kcache, vcache, sm_scale: float, stream=None):
        """Decode attention over the page table written by select()."""
        msa_sparse_attn_decode(self.rows, self.G, self.D, q, kcache, vcache, self.D, self.Hkv * self.D,
                               self.page_table, self.k, self.row_len, sm_scale, self.out, self.lse, self.ws, stream)

    def select_attend(self, q, kcache, vcache, sm_scale: float, stream=None):
        """Top-k, page table and attention from the scores, in the way ``select_mode`` says."""
        if self.select_mode == "attend":
            msa_topk_attn_decode(self.batch, self.scores, self.k, kcache, vcache, self.G, q, sm_scale, self.sel,
                                 self.cnt, self.page_table, self.row_len, self.out, self.lse, self.ws, stream)
        else:
            self.select(kcache, stream)
            self.attend(q, kcache, vcache, sm_scale, stream)

    def __call__(self, q, q_idx, kcache, vcache, kidx, sm_scale: float, stream=None):
        self.score(q_idx, kidx, stream)
        self.select_attend(q, kcache, vcache, sm_scale, stream)
        return self.out, self.lse


class MSAPrefill:
    """``fused=True`` scores and selects in one call (msa_index_topk): for k <= 16 the block scores
    never reach memory and ``scores`` is not kept; on the long-prefill workload this is faster than
    the two calls.  ``fused=False`` runs msa_index_score then msa_topk_blocks and keeps the scores.
    ``fused=None`` (the default) takes the fused call when its launch fills the chip, i.e. has at
    least ``FUSED_MIN_WGS`` workgroups of 256 query rows per KV head; shorter chunks take the
    two calls, whose scorer splits each row tile's blocks over several workgroups."""

    ROW_TILE = 256        # query rows per four-wave workgroup of the prefill scorer
    FUSED_MIN_WGS = 256   # half of the two four-wave workgroups per CU (the scorer takes eight-wave
                          # workgroups of 512 rows, one per CU, from 512 such workgroups on)
    # msa_sparse_attn_prefill's query-tile path (tile_min_rows > 0) merges partials on chip; on the long
    # prefill it cuts the merge from 1.6 to 0.9 ms but its attention is slower than the per-block kernel's,
    # so by default every selected block keeps its own partial
    TILE_MIN_ROWS = 0

    @classmethod
    def prefers_fused(cls, num_queries: int, Hkv: int) -> bool:
        """The default route: the fused call when its launch has FUSED_MIN_WGS workgroups or more."""
        return -(-num_queries // cls.ROW_TILE) * Hkv >= cls.FUSED_MIN_WGS

    def __init__(self, batch: Batch, Hkv: int, G: int, D: int, k: int, num_pages: int, device="cuda",
                 fused=None, tile_min_rows=None):
        Nq, mb = batch.num_queries, batch.max_blocks
        self.batch, self.Hkv, self.G, self.D, self.k, self.num_pages = batch, Hkv, G, D, k, num_pages
        self.tile_min_rows = self.TILE_MIN_ROWS if tile_min_rows is None else int(tile_min_rows)
        self.fused = self.prefers_fused(Nq, Hkv) if fused is None else bool(fused)
        self.scores = None if self.fused else torch.empty((Nq, Hkv, mb), dtype=torch.float32, device=device)
        self.topk_ws = torch.empty((max(1, msa_index_topk_workspace_size(batch, Hkv, k)),), dtype=torch.uint8,
                                   device=device)
        self.sel = torch.empty((Nq, Hkv, k), dtype=torch.int32, device=device)
        self.cnt = torch.empty((Nq, Hkv), dtype=torch.int32, device=device)
        self.part_o = torch.empty((Nq, Hkv, k, G, D), dtype=torch.bfloat16, device=device)
        self.part_lse = torch.empty((Nq, Hkv, k, G), dtype=torch.float32, device=device)
        self.out = torch.empty((Nq, Hkv * G, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((Nq, Hkv * G), dtype=torch.float32, device=device)
        self.ws = torch.empty((msa_sparse_attn_prefill_workspace_size(batch, Hkv, k),), dtype=torch.uint8,
                              device=device)

    def score(self, q_idx, kidx, stream=None):
        if self.fused:
            msa_index_topk(self.batch, q_idx, kidx, self.k, self.sel, self.cnt, self.topk_ws, stream)
        else:
            msa_index_score(self.batch, q_idx, kidx, self.scores, stream)

    def select(self, stream=None):
        if not self.fused:
            msa_topk_blocks(self.batch, self.Hkv, self.scores, self.k, self.sel, self.cnt, stream)

    def attend(self, q, kcache, vcache, sm_scale: float, stream=None):
        msa_sparse_attn_prefill(self.batch, self.G, q, kcache, vcache, self.sel, self.cnt, self.k, sm_scale,
                                self.part_o, self.part_lse, self.ws, stream, tile_min_rows=self.tile_min_rows)

    def merge(self, stream=None):
        rows = self.batch.num_queries * self.Hkv
        msa_lse_merge(rows, self.k, self.G, self.D, self.part_o, self.part_lse, self.out, self.lse, stream)

    def merge_bytes(self) -> int:
        """Bytes the merge moves: every part slot's partial and LSE in, the outputs out."""
        return (self.part_o.numel() * 2 + self.part_lse.numel() * 4 + self.out.numel() * 2 + self.lse.numel() * 4)

    def __call__(self, q, q_idx, kcache, vcache, kidx, sm_scale: float, stream=None):
        self.score(q_idx, kidx, stream)
        self.select(stream)
        self.attend(q, kcache, vcache, sm_scale, stream)
        self.merge(stream)
        return self.out, self.lse


class MSAPrefillQueryMajor:
    """Prefill attention query-major, for A/B against ``MSAPrefill``: the selection is turned into a
    per-row page table (ascending blocks, so only the diagonal block is partial) and each row reads
    its k blocks itself.  Same outputs as ``MSAPrefill`` up to rounding (bf16 partials there)."""

    def __init__(self, batch: Batch, Hkv: int, G: int, D: int, k: int, num_pages: int, device="cuda"):
        Nq, mb = batch.num_queries, batch.max_blocks
        self.batch, self.Hkv, self.G, self.D, self.k, self.num_pages = batch, Hkv, G, D, k, num_pages
        self.rows = Nq * Hkv
        self.scores = torch.empty((Nq, Hkv, mb), dtype=torch.float32, device=device)
        self.sel = torch.empty((Nq, Hkv, k), dtype=torch.int32, device=device)
        self.cnt = torch.empty((Nq, Hkv), dtype=torch.int32, device=device)
        self.page_table = torch.empty((self.rows, k), dtype=torch.int32, device=device)
        self.row_len = torch.empty((self.rows,), dtype=torch.int32, device=device)
        self.out = torch.empty((Nq, Hkv * G, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((Nq, Hkv * G), dtype=torch.float32, device=device)
        ws = msa_sparse_attn_decode_workspace_size(self.rows, G, D, k)
        self.ws = torch.zeros((ws,), dtype=torch.uint8, device=device) if ws else None

    def score(self, q_idx, kidx, stream=None):
        msa_index_score(self.batch, q_idx, kidx, self.scores, stream)

    def select(self, kcache, stream=None):
        msa_topk_page_table(self.batch, kcache, self.scores, self.k, self.sel, self.cnt, self.page_table,
                            self.row_len, stream)

    def attend(self, q, kcache, vcache, sm_scale: float, stream=None):
        msa_sparse_attn_decode(self.rows, self.G, self.D, q, kcache, vcache, self.D, self.Hkv * self.D,
                               self.page_table, self.k, self.row_len, sm_scale, self.out, self.lse, self.ws, stream)

    def __call__(self, q, q_idx, kcache, vcache, kidx, sm_scale: float, stream=None):
        self.score(q_idx, kidx, stream)
        self.select(kcache, stream)
        self.attend(q, kcache, vcache, sm_scale, stream)
        return self.out, self.lse
