"""GPU test plumbing: build device inputs, call the library, bring results back."""
from __future__ import annotations

import sys

import numpy as np
import torch

import msa_inputs as mi


def lib():
    """The HIP binding; raises if libmsa.so is missing (no fallback)."""
    import block_sparse_long_msa_amd as msa
    msa.load()
    return msa


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def setup(wl: mi.Workload, on_gpu_generation: bool = False, host_copy: bool = False):
    """(device inputs, cpu inputs or None).  Small cases are drawn on the CPU and copied; long ones can
    be drawn on the GPU (CPU normal draws of hundreds of millions of values take minutes), with an
    optional host copy of exactly those values for the oracle."""
    if on_gpu_generation:
        dev = mi.make_inputs(wl, "cuda")
        return dev, (dev.to("cpu") if host_copy else None)
    cpu = mi.make_inputs(wl, "cpu")
    return cpu.to("cuda"), cpu


def batch(dev, max_q=None):
    msa = lib()
    if max_q is None:
        max_q = int(max(dev.wl.q_counts))
    return msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max_q)


def nan_f32(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def poison_i32(*shape):
    return torch.full(shape, -7777, dtype=torch.int32, device="cuda")


def scores(dev, b):
    wl = dev.wl
    s = nan_f32(wl.Nq, wl.Hkv, dev.block_table.shape[1])
    lib().msa_index_score(b, dev.q_idx, dev.kidx, s)
    return s


def topk(dev, b, s, k=None):
    wl = dev.wl
    k = k or wl.k
    sel = poison_i32(wl.Nq, wl.Hkv, k)
    cnt = poison_i32(wl.Nq, wl.Hkv)
    lib().msa_topk_blocks(b, wl.Hkv, s, k, sel, cnt)
    return sel, cnt


def page_table(dev, b, sel, cnt, k=None):
    wl = dev.wl
    k = k or wl.k
    pt = poison_i32(wl.Nq * wl.Hkv, k)
    rl = poison_i32(wl.Nq * wl.Hkv)
    lib().msa_build_sparse_page_table(b, dev.kcache, sel, cnt, k, pt, rl)
    return pt, rl


def topk_page_table(dev, b, s, k=None):
    """msa_topk_page_table: top-k and the page table in one call."""
    wl = dev.wl
    k = k or wl.k
    sel, cnt = poison_i32(wl.Nq, wl.Hkv, k), poison_i32(wl.Nq, wl.Hkv)
    pt, rl = poison_i32(wl.Nq * wl.Hkv, k), poison_i32(wl.Nq * wl.Hkv)
    lib().msa_topk_page_table(b, dev.kcache, s, k, sel, cnt, pt, rl)
    return sel, cnt, pt, rl


def decode_attention(dev, pt, rl, k=None):
    wl = dev.wl
    k = k or wl.k
    msa = lib()
    rows = wl.Nq * wl.Hkv
    out = torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = nan_f32(wl.Nq, wl.Hq)
    ws = torch.zeros(msa.msa_sparse_attn_decode_workspace_size(rows, wl.G, wl.D, k), dtype=torch.uint8,
                     device="cuda")
    msa.msa_sparse_attn_decode(rows, wl.G, wl.D, dev.q, dev.kcache, dev.vcache, wl.D, wl.Hkv * wl.D, pt, k, rl,
                               dev.scale, out, lse, ws)
    return out, lse


def topk_attn_decode(dev, b, s, k=None):
    """msa_topk_attn_decode: top-k, page table and decode attention in one call.  Returns
    (sel, cnt, page_table, row_len, out, lse), every buffer poisoned beforehand."""
    wl = dev.wl
    k = k or wl.k
    msa = lib()
    rows = wl.Nq * wl.Hkv
    sel, cnt = poison_i32(wl.Nq, wl.Hkv, k), poison_i32(wl.Nq, wl.Hkv)
    pt, rl = poison_i32(rows, k), poison_i32(rows)
    out = torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = nan_f32(wl.Nq, wl.Hq)
    ws = torch.zeros(msa.msa_sparse_attn_decode_workspace_size(rows, wl.G, wl.D, k), dtype=torch.uint8,
                     device="cuda")
    msa.msa_topk_attn_decode(b, s, k, dev.kcache, dev.vcache, wl.G, dev.q, dev.scale, sel, cnt, pt, rl, out, lse, ws)
    return sel, cnt, pt, rl, out, lse


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


class DeviceView:
    """Read-only indexable view of a GPU tensor for the oracle: every index copies just that slice
    to the host as float32 (bf16 upcast exactly).  Lets the oracle work one output at a time
    on caches far larger than host memory wants to hold."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        if isinstance(idx, np.ndarray):
            idx = torch.from_numpy(idx).to(self.t.device)
        v = self.t[idx]
        return (v.float() if v.is_floating_point() else v).cpu().numpy()


def prefill(dev, b, sel, cnt, k=None, tile_min=0, slot_of=None):
    """KV-block-major attention partials (tile_min_rows = tile_min), then the LSE merge."""
    wl = dev.wl
    k = k or wl.k
    msa = lib()
    po = torch.full((wl.Nq, wl.Hkv, k, wl.G, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    pl = nan_f32(wl.Nq, wl.Hkv, k, wl.G)
    ws = torch.empty(msa.msa_sparse_attn_prefill_workspace_size(b, wl.Hkv, k), dtype=torch.uint8, device="cuda")
    msa.msa_sparse_attn_prefill(b, wl.G, dev.q, dev.kcache, dev.vcache, sel, cnt, k, dev.scale, po, pl, ws,
                                tile_min_rows=tile_min, slot_of=slot_of)
    out = torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = nan_f32(wl.Nq, wl.Hq)
    msa.msa_lse_merge(wl.Nq * wl.Hkv, k, wl.G, wl.D, po, pl, out, lse)
    return po, pl, out, lse
