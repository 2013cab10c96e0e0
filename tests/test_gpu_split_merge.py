"""The decode split merge inside the attention launch: the last split of a row to finish folds the
row's partials, found through one arrival counter per row at the end of the workspace.

Checked here: outputs match the oracle and a run on a fresh zeroed workspace bit for bit; every call
leaves the counters at zero; the partial region needs no clearing (it is poisoned between calls);
one workspace serves calls of different row counts and split counts in turn; partials left by a call
on other inputs never leak into the next call's output.  Both routes are covered: the fused top-k +
attention launch (msa_topk_attn_decode) and the page-table attention (msa_sparse_attn_decode).
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _gpu import announce, batch, host, lib, nan_f32, poison_i32, scores, setup, topk_page_table
from _helpers import assert_attn_close, np_inputs

pytestmark = pytest.mark.gpu

CASES = {
    # 24 rows -> 8 splits of one page; the 777-token request has 7 blocks, so its rows' last split is empty
    "rows24_splits8": dict(ctx=[5000, 2049, 777], nq=[1, 3, 2], Hq=32, Hkv=4, D=128, Di=128, k=8),
    # one row -> 64 splits, merged in eight batches of eight parts
    "one_row_splits64": dict(ctx=[9000], nq=[1], Hq=16, Hkv=1, D=64, Di=64, k=64),
    # 64 rows -> 4 splits of four pages, the agentic decode's split shape at a smaller context
    "rows64_splits4": dict(ctx=[3000] * 8, nq=[1] * 8, Hq=64, Hkv=8, D=128, Di=128, k=16),
}


def _wl(name, seed):
    c = dict(CASES[name])
    ctx, nq = c.pop("ctx"), c.pop("nq")
    return mi.small_workload(ctx, nq, seed=seed, **c)


def _counter_region(ws, rows):
    end = ws.numel() & ~255
    return ws[end - (-(-rows * 4 // 256) * 256):end]


def _fused(dev, b, s, ws):
    wl = dev.wl
    rows = wl.Nq * wl.Hkv
    sel, cnt = poison_i32(wl.Nq, wl.Hkv, wl.k), poison_i32(wl.Nq, wl.Hkv)
    pt, rl = poison_i32(rows, wl.k), poison_i32(rows)
    out = torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = nan_f32(wl.Nq, wl.Hq)
    lib().msa_topk_attn_decode(b, s, wl.k, dev.kcache, dev.vcache, wl.G, dev.q, dev.scale, sel, cnt, pt, rl, out,
                               lse, ws)
    torch.cuda.synchronize()
    return out, lse, sel, cnt


def _paged(dev, pt, rl, ws):
    wl = dev.wl
    rows = wl.Nq * wl.Hkv
    out = torch.full((wl.Nq, wl.Hq, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = nan_f32(wl.Nq, wl.Hq)
    lib().msa_sparse_attn_decode(rows, wl.G, wl.D, dev.q, dev.kcache, dev.vcache, wl.D, wl.Hkv * wl.D, pt, wl.k, rl,
                                 dev.scale, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def _fresh_ws(wl):
    n = lib().msa_sparse_attn_decode_workspace_size(wl.Nq * wl.Hkv, wl.G, wl.D, wl.k)
    assert n > 0, "the case must split its rows"
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _same(a, b):
    return all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y) for x, y in zip(a, b))


@pytest.mark.parametrize("name", list(CASES))
def test_split_merge_matches_oracle_and_resets_counters(name):
    announce("split merge", name)
    dev, cpu = setup(_wl(name, seed=71))
    wl = dev.wl
    rows = wl.Nq * wl.Hkv
    b = batch(dev)
    s = scores(dev, b)
    ws = _fresh_ws(wl)
    out, lse, sel, cnt = _fused(dev, b, s, ws)
    assert torch.count_nonzero(_counter_region(ws, rows)).item() == 0, "counters not returned to zero"
    x = np_inputs(cpu)
    ref_o, ref_l = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           host(sel), host(cnt), wl.block, x.scale)
    assert_attn_close(host(out), ref_o, what="split-merged output")
    assert np.abs(host(lse) - ref_l).max() <= 1e-3

    # the partial region is poisoned (all-ones bytes: NaN floats) and the call repeated: same bits
    cr = _counter_region(ws, rows)
    body = ws[:ws.numel() - cr.numel() - (ws.numel() & 255)]
    body.fill_(255)
    again = _fused(dev, b, s, ws)
    assert _same((out, lse), again[:2]), "output depends on stale partial bytes"
    assert torch.count_nonzero(_counter_region(ws, rows)).item() == 0

    # the page-table route through the same workspace
    _, _, pt, rl = topk_page_table(dev, b, s)
    o2, l2 = _paged(dev, pt, rl, ws)
    assert _same((out, lse), (o2, l2)), "page-table route differs from the fused route"
    assert torch.count_nonzero(_counter_region(ws, rows)).item() == 0


def test_one_workspace_for_many_calls():
    """Calls of different row and split counts, and on different inputs, take turns on one buffer;
    each output equals that call's output on a fresh zeroed workspace."""
    announce("split merge: shared workspace")
    runs = []
    for name, seed in (("rows64_splits4", 81), ("rows24_splits8", 82), ("one_row_splits64", 83),
                       ("rows64_splits4", 84)):
        dev, _ = setup(_wl(name, seed))
        b = batch(dev)
        s = scores(dev, b)
        runs.append((dev, b, s, _fused(dev, b, s, _fresh_ws(dev.wl))))
    size = max(lib().msa_sparse_attn_decode_workspace_size(d.wl.Nq * d.wl.Hkv, d.wl.G, d.wl.D, d.wl.k)
               for d, _, _, _ in runs)
    ws = torch.zeros(size + 4096, dtype=torch.uint8, device="cuda")  # larger than any call needs
    for rep in range(3):
        for i, (dev, b, s, ref) in enumerate(runs):
            got = _fused(dev, b, s, ws)
            assert _same(ref, got), f"repeat {rep}, call {i}: differs from its fresh-workspace run"
