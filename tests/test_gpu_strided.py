"""Caches whose pages are spaced apart (msa_cache.page_stride): the K and V pages interleaved in one
pool [pages, 2, 128, Hkv, D], and the key-index cache with two pages' gap after every page.

Every call takes the strided views and must give the results of the same caches stored back to
back, bit for bit: the scores, the selections, the attention outputs and LSEs, the prefill partials.
The page tables follow the layout: an entry block_table[r, b] * 128 * Hkv + g of the back-to-back
cache becomes block_table[r, b] * (page_stride / D) + g.
"""
import copy

import pytest
import torch

import msa_inputs as mi
from _gpu import (announce, batch, decode_attention, lib, page_table, poison_i32, prefill, scores, setup, topk,
                  topk_attn_decode, topk_page_table)

pytestmark = pytest.mark.gpu

DECODE = {
    "gqa8_d128": dict(ctx=[3000, 1500, 777, 4100], nq=[1, 2, 1, 3], Hq=32, Hkv=4, D=128, Di=128, k=8,
                      hot_per_group=8),
    # rows split over several workgroups and merged: the page ids reach the split runs
    "split_d64": dict(ctx=[9000], nq=[1], Hq=8, Hkv=2, D=64, Di=64, k=32),
}
PREFILL = {
    "g4_d64": dict(ctx=[1700, 900], nq=[300, 140], Hq=8, Hkv=2, D=64, Di=64, k=4, hot_per_group=4,
                   hot_ref="centroid", q_idx_mode="centroid_mix"),
}


def _wl(c, seed):
    c = dict(c)
    ctx, nq = c.pop("ctx"), c.pop("nq")
    return mi.small_workload(ctx, nq, seed=seed, **c)


def _strided(dev):
    """The same inputs with K and V interleaved per page and a two-page gap after each key-index page."""
    sd = copy.copy(dev)
    kc, vc, ki = dev.kcache, dev.vcache, dev.kidx
    pool = torch.empty((kc.shape[0], 2) + tuple(kc.shape[1:]), dtype=kc.dtype, device=kc.device)
    pool[:, 0] = kc
    pool[:, 1] = vc
    sd.kcache, sd.vcache = pool[:, 0], pool[:, 1]
    ipool = torch.full((ki.shape[0], 3) + tuple(ki.shape[1:]), float("nan"), dtype=ki.dtype, device=ki.device)
    ipool[:, 1] = ki
    sd.kidx = ipool[:, 1]
    assert sd.kcache.stride(0) == 2 * kc[0].numel() and sd.kidx.stride(0) == 3 * ki[0].numel()
    return sd


def _same(a, b):
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _relayout(pt, wl, vps):
    """Back-to-back page ids (block * 128 * Hkv + g) in the strided layout (block * vps + g)."""
    g = pt % wl.Hkv
    blk = pt // (128 * wl.Hkv)
    return torch.where(pt >= 0, blk * vps + g, pt)


@pytest.mark.parametrize("name", list(DECODE))
def test_decode_on_strided_caches(name):
    announce("strided caches: decode", name)
    dev, _ = setup(_wl(DECODE[name], 13))
    sd = _strided(dev)
    wl = dev.wl
    vps = sd.kcache.stride(0) // wl.D
    b = batch(dev)
    s = scores(dev, b)
    s2 = scores(sd, b)
    assert _same(s, s2), "scores differ on the gapped key-index cache"
    ref = topk_attn_decode(dev, b, s)
    got = topk_attn_decode(sd, b, s)
    for n_, x, y in zip(("sel", "cnt"), got[:2], ref[:2]):
        assert _same(x, y), n_
    assert _same(got[2], _relayout(ref[2], wl, vps)), "page table does not follow the layout"
    assert _same(got[3], ref[3]) and _same(got[4], ref[4]) and _same(got[5], ref[5]), "attention differs"
    # the separate route: top-k + page table, then attention through the views
    sel, cnt, pt, rl = topk_page_table(sd, b, s)
    assert _same(pt, got[2]) and _same(rl, got[3])
    sel2, cnt2 = topk(dev, b, s)
    pt2, rl2 = page_table(sd, b, sel2, cnt2)
    assert _same(pt2, pt) and _same(rl2, rl)
    out, lse = decode_attention(sd, pt, rl)
    out_c, lse_c = decode_attention(dev, ref[2], ref[3])
    assert _same(out, out_c) and _same(lse, lse_c)
    # the allocation-free entry point on the same views
    rows = wl.Nq * wl.Hkv
    bufs = (poison_i32(wl.Nq, wl.Hkv, wl.k), poison_i32(wl.Nq, wl.Hkv), poison_i32(rows, wl.k), poison_i32(rows),
            torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda"),
            torch.full((wl.Nq, wl.Hq), float("nan"), dtype=torch.float32, device="cuda"))
    lib().msa_topk_attn_decode_noalloc(b, s, wl.k, sd.kcache, sd.vcache, wl.G, dev.q, dev.scale, *bufs)
    torch.cuda.synchronize()
    for x, y in zip(bufs, got):
        assert _same(x, y), "allocation-free route differs on the strided caches"


@pytest.mark.parametrize("name", list(PREFILL))
@pytest.mark.parametrize("tile_min", [0, 8])
def test_prefill_on_strided_caches(name, tile_min):
    announce("strided caches: prefill", name, f"tile_min_rows={tile_min}")
    dev, _ = setup(_wl(PREFILL[name], 17))
    sd = _strided(dev)
    wl = dev.wl
    b = batch(dev)
    msa = lib()
    s, s2 = scores(dev, b), scores(sd, b)
    assert _same(s, s2), "prefill scores differ on the gapped key-index cache"
    sel, cnt = topk(dev, b, s)
    for d in (dev, sd):  # the fused scorer + top-k reads the gapped cache as well
        fs, fc = poison_i32(wl.Nq, wl.Hkv, wl.k), poison_i32(wl.Nq, wl.Hkv)
        ws = torch.empty(max(1, msa.msa_index_topk_workspace_size(b, wl.Hkv, wl.k)), dtype=torch.uint8, device="cuda")
        msa.msa_index_topk(b, d.q_idx, d.kidx, wl.k, fs, fc, ws)
        assert _same(fs, sel) and _same(fc, cnt)
    ref = prefill(dev, b, sel, cnt, tile_min=tile_min)
    got = prefill(sd, b, sel, cnt, tile_min=tile_min)
    for n_, x, y in zip(("part_o", "part_lse", "out", "lse"), got, ref):
        if n_ == "part_o":  # slots a row never wrote keep their poison: compare where the LSE is set
            keep = torch.isfinite(ref[1]).unsqueeze(-1).expand_as(x)
            assert torch.equal(x.view(torch.int16)[keep], y.view(torch.int16)[keep]), n_
        else:
            assert _same(x, y), n_


def test_strided_views_are_rejected_when_rows_are_not_contiguous():
    """Only the page dimension may be strided: a head-major view is refused by the binding."""
    dev, _ = setup(_wl(DECODE["gqa8_d128"], 19))
    b = batch(dev)
    s = scores(dev, b)
    wl = dev.wl
    bad = dev.kcache.transpose(1, 2).contiguous().transpose(1, 2)  # [P, 128, H, D] view of [P, H, 128, D]
    with pytest.raises(ValueError, match="contiguous"):
        lib().msa_topk_page_table(b, bad, s, wl.k, poison_i32(wl.Nq, wl.Hkv, wl.k), poison_i32(wl.Nq, wl.Hkv),
                                  poison_i32(wl.Nq * wl.Hkv, wl.k), poison_i32(wl.Nq * wl.Hkv))
