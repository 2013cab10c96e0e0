"""K/V caches offloaded to pinned host memory while the key-index cache stays in HBM: the scorer and
top-k run on device memory, and decode attention reads only the selected blocks over the host link.

Same kernels, same bytes: the outputs must equal the all-in-HBM run bit for bit, and the oracle
within the attention tolerance.
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _gpu import announce, batch, decode_attention, host, lib, scores, setup, topk_page_table
from _helpers import assert_attn_close, np_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ctx,nq,Hq,Hkv,D,k", [
    ([5000, 2049, 777, 12345], [1, 1, 1, 1], 64, 8, 128, 16),   # one token per request, 4 splits per row
    ([3000, 900], [4, 2], 16, 2, 64, 5),                         # several tokens per request, D = 64
])
def test_decode_with_kv_on_host(ctx, nq, Hq, Hkv, D, k):
    msa = lib()
    wl = mi.small_workload(ctx, nq, Hq=Hq, Hkv=Hkv, D=D, Di=D, k=k, seed=41)
    announce("offload", wl.name)
    dev, cpu = setup(wl)
    x = np_inputs(cpu)
    b = batch(dev)
    s = scores(dev, b)
    sel, cnt, pt, rl = topk_page_table(dev, b, s)
    out_d, lse_d = decode_attention(dev, pt, rl)

    kh = msa.HostResident(dev.kcache.cpu().pin_memory())
    vh = msa.HostResident(dev.vcache.cpu().pin_memory())
    rows = wl.Nq * wl.Hkv
    out_h = torch.full_like(out_d, float("nan"))
    lse_h = torch.full_like(lse_d, float("nan"))
    ws_n = msa.msa_sparse_attn_decode_workspace_size(rows, wl.G, wl.D, wl.k)
    ws = torch.zeros(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None
    msa.msa_sparse_attn_decode(rows, wl.G, wl.D, dev.q, kh, vh, wl.D, wl.Hkv * wl.D, pt, wl.k, rl, dev.scale,
                               out_h, lse_h, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_h.view(torch.int16), out_d.view(torch.int16))
    assert torch.equal(lse_h, lse_d)

    sel, cnt = host(sel), host(cnt)
    ref_o, ref_l = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, wl.block, x.scale)
    assert_attn_close(host(out_h), ref_o, what="attention with K/V on the host")
    assert np.abs(host(lse_h) - ref_l).max() <= 1e-3


def test_host_resident_rejects_device_and_unpinned():
    msa = lib()
    with pytest.raises(ValueError):
        msa.HostResident(torch.zeros(4, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        msa.HostResident(torch.zeros(4, dtype=torch.bfloat16))
