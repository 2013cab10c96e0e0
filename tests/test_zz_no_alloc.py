"""msa_topk_attn_decode_noalloc, the allocation-free form of msa_topk_attn_decode for callers that cannot
allocate (graph capture, serving loops): called through the C ABI twice in a row -- the second batch
smaller than the first, so the shared static scratch still holds the first call's partials -- and each
time bit-identical to msa_topk_attn_decode with a workspace on the same inputs (six outputs).  Both
batches are small enough that rows are split over workgroups, so the scratch is in use."""
import pytest
import torch

import msa_inputs as mi
from _gpu import announce, batch, lib, nan_f32, poison_i32, scores, setup, topk_attn_decode

pytestmark = pytest.mark.gpu


def _noalloc(dev, b, s):
    wl = dev.wl
    rows = wl.Nq * wl.Hkv
    sel, cnt = poison_i32(wl.Nq, wl.Hkv, wl.k), poison_i32(wl.Nq, wl.Hkv)
    pt, rl = poison_i32(rows, wl.k), poison_i32(rows)
    out = torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = nan_f32(wl.Nq, wl.Hq)
    lib().msa_topk_attn_decode_noalloc(b, s, wl.k, dev.kcache, dev.vcache, wl.G, dev.q, dev.scale, sel, cnt, pt, rl,
                                       out, lse)
    return sel, cnt, pt, rl, out, lse


def test_noalloc_equals_workspace_route_on_two_calls():
    msa = lib()
    large = mi.small_workload([20000, 9000, 30001, 5000, 12345, 7000, 15000, 20001], [1] * 8, Hq=64, Hkv=8, D=128,
                              Di=128, k=16, seed=5, hot_per_group=16)
    small = mi.small_workload([3000, 700], [1, 2], Hq=32, Hkv=4, D=128, Di=128, k=8, seed=6)
    for wl in (large, small):
        announce("noalloc", wl.name, f"rows={wl.Nq * wl.Hkv}")
        rows = wl.Nq * wl.Hkv
        need = msa.msa_sparse_attn_decode_workspace_size(rows, wl.G, wl.D, wl.k)
        assert 0 < need <= (4 << 20), "the case must use the split scratch"
        dev, _ = setup(wl)
        b = batch(dev)
        s = scores(dev, b)
        ref = topk_attn_decode(dev, b, s)
        got = _noalloc(dev, b, s)
        torch.cuda.synchronize()
        for name, a, f in zip(("sel", "cnt", "page_table", "row_len", "out", "lse"), ref, got):
            assert torch.equal(a, f), f"{wl.name}: {name} differs from msa_topk_attn_decode"
