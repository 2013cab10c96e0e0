"""Seeded synthetic inputs for MiniMax Sparse Attention (MSA).

This module only draws numbers: paged caches, block tables, queries and query
index vectors shaped like the workloads the MSA serving write-ups describe
(128-token paged blocks, 60K-token agentic prefixes at concurrency 8, a 32K-token
prefill chunk over a 96K prefix, 1M-token contexts, ragged concurrent decode).
It computes nothing the method computes, so both the CPU oracle (``oracle/``)
and the HIP library tests can take their inputs from here.

Recipe (the same for every workload):
  * Structure (context lengths, the physical page permutation, hot blocks,
    cluster choices, tie copies) is drawn with NumPy ``PCG64(seed)`` on the host,
    so it is identical for a seed whatever the device.
  * Bulk values are N(0,1) fp32 draws from a ``torch.Generator`` seeded with
    ``seed`` on the target device, rounded once to bf16 (round to nearest even).
    Small cases are drawn on the CPU and copied, so both sides see the same bytes.
  * Caches are ``[pages, 128, Hkv, D]`` bf16; the block table maps logical block
    b of request r to a physical page; unused block-table entries hold page 0
    (never read by a correct kernel, and always a valid address).
  * The query tokens of request r are its last ``nq_r`` cache tokens, so query
    j of request r sits at position ``L_r - nq_r + j`` and its key/value and
    key-index rows are already in the cache (the decode token is written before
    scoring).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

BLOCK = 128


@dataclasses.dataclass
class Workload:
    """Shape of one synthetic MSA invocation."""

    name: str
    ctx_lens: List[int]          # L_r: tokens in request r's cache, current tokens included
    q_counts: List[int]          # new (query) tokens per request
    Hq: int = 64
    Hkv: int = 8
    D: int = 128
    Di: int = 128
    k: int = 16
    block: int = BLOCK
    hot_per_group: int = 0       # planted hot blocks per (request, KV group)
    hot_ref: str = "query"       # "query": bias is 0.5*q_idx of the request's last query; "centroid": 0.5*c_g
    q_idx_mode: str = "normal"   # "normal" | "centroid_mix" ((z + c_g)/sqrt2) | "clusters"
    n_clusters: int = 64
    cluster_noise: float = 0.1
    tie_frac: float = 0.0        # fraction of full blocks per (r, g) given a bitwise copy of another block's k_idx
    extra_pages: int = 0         # unused pages in the pool
    seed: int = 1000

    @property
    def B(self) -> int:
        return len(self.ctx_lens)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def Nq(self) -> int:
        return int(sum(self.q_counts))

    def nblocks(self, r: int) -> int:
        return -(-self.ctx_lens[r] // self.block)

    @property
    def max_blocks(self) -> int:
        return max(self.nblocks(r) for r in range(self.B))

    @property
    def num_pages(self) -> int:
        return sum(self.nblocks(r) for r in range(self.B)) + self.extra_pages


# --- the five workloads ------------------------------------------------------

def tiny_prefill(seed: int = 1000) -> Workload:
    """One 2048-token sequence prefilled at once (16 blocks), Hq=8, Hkv=2, D=Di=64, top-4,
    four planted hot blocks per group biased by 0.5*c_g with q_idx = (z + c_g)/sqrt(2)."""
    return Workload("tiny_prefill_2k", ctx_lens=[2048], q_counts=[2048], Hq=8, Hkv=2, D=64, Di=64,
                    k=4, hot_per_group=4, hot_ref="centroid", q_idx_mode="centroid_mix", seed=seed)


def agentic_decode(seed: int = 1001, batch: int = 8) -> Workload:
    """Batch 8, 61440-token prefix + 1 new token each (481 blocks, last holds 1 token),
    Hq=64, Hkv=8, D=Di=128, top-16, 16 hot blocks per (request, group)."""
    return Workload("agentic_decode_b8_61k", ctx_lens=[61441] * batch, q_counts=[1] * batch,
                    k=16, hot_per_group=16, hot_ref="query", seed=seed)


def spec_decode(seed: int = 1005, batch: int = 8, draft: int = 4) -> Workload:
    """Multi-token decode (speculative verification): the agentic decode with `draft` query tokens per
    request (the last `draft` tokens of a 61440 + `draft` context), each scoring, selecting and
    attending on its own causal range; 16 hot blocks per (request, group)."""
    return Workload(f"spec_decode_b{batch}_x{draft}_61k", ctx_lens=[61440 + draft] * batch, q_counts=[draft] * batch,
                    k=16, hot_per_group=16, hot_ref="query", seed=seed)


def long_prefill(seed: int = 1002, new_tokens: int = 32768, prefix: int = 98304) -> Workload:
    """32768 new tokens over a 98304-token cached prefix (131072 total, 1024 blocks), top-16,
    q_idx drawn from 64 per-group centroids plus N(0, 0.1^2) noise."""
    return Workload("long_prefill_32k_over_96k", ctx_lens=[prefix + new_tokens], q_counts=[new_tokens],
                    k=16, q_idx_mode="clusters", seed=seed)


def million_decode(seed: int = 1003, batch: int = 1) -> Workload:
    """1,048,576-token context (8192 blocks), batch 1 or 4, top-32, 32 hot blocks."""
    return Workload(f"million_decode_b{batch}_1m", ctx_lens=[1 << 20] * batch, q_counts=[1] * batch,
                    k=32, hot_per_group=32, hot_ref="query", seed=seed)


def ragged_lengths(n: int, seed: int, median: int = 32768, sigma: float = 1.0,
                   lo: int = 4096, hi: int = 262144) -> List[int]:
    """Log-normal context lengths clipped to [lo, hi] and kept off multiples of 128."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    out = []
    for x in rng.normal(math.log(median), sigma, size=n):
        L = int(min(max(round(math.exp(x)), lo), hi))
        if L % BLOCK == 0:
            L = L - 1 if L >= hi else L + 1
        out.append(L)
    return out


def ragged_decode(seed: int = 1004, batch: int = 96) -> Workload:
    """96 requests with log-normal contexts (median 32K, 4K..256K, never a multiple of 128),
    top-16, ties planted in 1% of full blocks per (request, group)."""
    return Workload("ragged_decode_96", ctx_lens=ragged_lengths(batch, seed), q_counts=[1] * batch,
                    k=16, tie_frac=0.01, seed=seed)


WORKLOADS = {
    "tiny_prefill": tiny_prefill,
    "agentic_decode": agentic_decode,
    "long_prefill": long_prefill,
    "million_decode": million_decode,
    "ragged_decode": ragged_decode,
    "spec_decode": spec_decode,
}


# --- drawing -----------------------------------------------------------------

@dataclasses.dataclass
class Inputs:
    wl: Workload
    kcache: torch.Tensor       # [P, BS, Hkv, D] bf16
    vcache: torch.Tensor       # [P, BS, Hkv, D] bf16
    kidx: torch.Tensor         # [P, BS, Hkv, Di] bf16
    block_table: torch.Tensor  # [B, max_blocks] int32
    ctx_len: torch.Tensor      # [B] int32
    cu_q: torch.Tensor         # [B+1] int32
    q_pos: torch.Tensor        # [Nq] int32
    q_req: torch.Tensor        # [Nq] int32 (derived from cu_q, for convenience)
    q: torch.Tensor            # [Nq, Hq, D] bf16
    q_idx: torch.Tensor        # [Nq, Hkv, Di] bf16
    hot: dict                  # (r, g) -> sorted list of planted hot blocks
    ties: dict                 # (r, g) -> list of (dst_block, src_block) bitwise copies

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.wl.D)

    def to(self, device) -> "Inputs":
        kw = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for name, v in kw.items():
            if isinstance(v, torch.Tensor):
                kw[name] = v.to(device)
        return Inputs(**kw)


def _normal(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_inputs(wl: Workload, device="cpu") -> Inputs:
    """Draw every tensor of ``wl`` on ``device`` (see the module docstring for the recipe)."""
    device = torch.device(device)
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    B, BS, Hkv = wl.B, wl.block, wl.Hkv

    # physical pages: a seeded permutation of the pool
    P = wl.num_pages
    perm = rng.permutation(P).astype(np.int32)
    bt = np.zeros((B, wl.max_blocks), dtype=np.int32)
    o = 0
    for r in range(B):
        nb = wl.nblocks(r)
        bt[r, :nb] = perm[o:o + nb]
        o += nb
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(wl.q_counts)
    pos = np.concatenate([np.arange(L - n, L, dtype=np.int32) for L, n in zip(wl.ctx_lens, wl.q_counts)])
    req = np.repeat(np.arange(B, dtype=np.int32), wl.q_counts)

    # bulk N(0,1) values, drawn in a fixed order
    kcache = _normal(gen, (P, BS, Hkv, wl.D), device)
    vcache = _normal(gen, (P, BS, Hkv, wl.D), device)
    kidx = _normal(gen, (P, BS, Hkv, wl.Di), device)
    q = _normal(gen, (wl.Nq, wl.Hq, wl.D), device)

    centroids = None
    if wl.q_idx_mode == "normal":
        q_idx = _normal(gen, (wl.Nq, Hkv, wl.Di), device)
    elif wl.q_idx_mode == "centroid_mix":
        centroids = _normal(gen, (Hkv, wl.Di), device)
        z = _normal(gen, (wl.Nq, Hkv, wl.Di), device)
        q_idx = (z + centroids[None]) / math.sqrt(2.0)
    elif wl.q_idx_mode == "clusters":
        cents = _normal(gen, (Hkv, wl.n_clusters, wl.Di), device)
        choice = torch.from_numpy(rng.integers(0, wl.n_clusters, size=(wl.Nq, Hkv))).to(device)
        gidx = torch.arange(Hkv, device=device)[None, :].expand(wl.Nq, Hkv)
        noise = _normal(gen, (wl.Nq, Hkv, wl.Di), device)
        q_idx = cents[gidx, choice] + wl.cluster_noise * noise
    else:
        raise ValueError(wl.q_idx_mode)

    # planted hot blocks: every k_idx row of the block gets +0.5 * reference direction
    hot = {}
    if wl.hot_per_group:
        for r in range(B):
            full = wl.ctx_lens[r] // BS          # complete blocks of request r
            last_q = int(cu[r + 1]) - 1
            for g in range(Hkv):
                hb = np.sort(rng.choice(full, size=min(wl.hot_per_group, full), replace=False))
                hot[(r, g)] = [int(b) for b in hb]
                ref = centroids[g] if wl.hot_ref == "centroid" else q_idx[last_q, g]
                pages = torch.from_numpy(bt[r, hb].astype(np.int64)).to(device)
                kidx[pages, :, g, :] += 0.5 * ref
    # round once to bf16
    kcache = kcache.to(torch.bfloat16)
    vcache = vcache.to(torch.bfloat16)
    kidx = kidx.to(torch.bfloat16)
    q = q.to(torch.bfloat16)
    q_idx = q_idx.to(torch.bfloat16)

    # ties: bitwise copies of another full block's k_idx rows for that group
    ties = {}
    if wl.tie_frac > 0:
        for r in range(B):
            full = wl.ctx_lens[r] // BS
            if full < 2:
                continue  # a tie needs two full blocks
            nt = min(max(1, int(round(wl.tie_frac * full))), full // 2)
            for g in range(Hkv):
                pairs = []
                picks = rng.choice(full, size=2 * nt, replace=False)
                for dst, src in zip(picks[:nt], picks[nt:]):
                    kidx[int(bt[r, dst]), :, g, :] = kidx[int(bt[r, src]), :, g, :]
                    pairs.append((int(dst), int(src)))
                ties[(r, g)] = pairs

    t = lambda a: torch.from_numpy(a).to(device)
    return Inputs(wl=wl, kcache=kcache, vcache=vcache, kidx=kidx, block_table=t(bt),
                  ctx_len=t(np.asarray(wl.ctx_lens, dtype=np.int32)), cu_q=t(cu), q_pos=t(pos),
                  q_req=t(req), q=q, q_idx=q_idx, hot=hot, ties=ties)


def small_workload(ctx_lens, q_counts, Hq=8, Hkv=2, D=64, Di=64, k=4, seed=7, **kw) -> Workload:
    """A free-form small workload for tests (block size 128 unless given)."""
    return Workload(f"small_{seed}", ctx_lens=list(ctx_lens), q_counts=list(q_counts), Hq=Hq, Hkv=Hkv,
                    D=D, Di=Di, k=k, seed=seed, **kw)


def random_partials(rows: int, parts: int, G: int, D: int, seed: int, empty_frac: float = 0.2,
                    device="cpu"):
    """Random per-block partial outputs (bf16) and log-sum-exps (fp32, -inf for empty slots)
    for exercising the merge on its own. Slot 0 of every row is always present."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    po = torch.randn((rows, parts, G, D), generator=gen, device=device).to(torch.bfloat16)
    pl = 4.0 * torch.randn((rows, parts, G), generator=gen, device=device)
    drop = torch.rand((rows, parts), generator=gen, device=device) < empty_frac
    drop[:, 0] = False
    pl = torch.where(drop[:, :, None], torch.full_like(pl, float("-inf")), pl)
    return po, pl
