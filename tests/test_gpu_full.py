"""Full-size parity: the five workloads at their full sizes, run through the same pipeline objects
(and so the same launch configuration) that bench.py times.

The oracle computes sampled outputs one by one (whole requests or evenly spaced query rows; every
KV head; all candidate blocks unless stated), reading the caches slice by slice from the GPU.
Properties that hold at any size are checked on every row: top-k bit-exact against the oracle's
top-k of the GPU's own scores, the page table bit-exact, counts and padding, finite outputs.
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _gpu import DeviceView, announce, host, lib
from _helpers import assert_attn_close, selection_excused

pytestmark = pytest.mark.gpu


def _decode_run(dev):
    msa = lib()
    from block_sparse_long_msa_amd.pipeline import MSADecode
    wl = dev.wl
    b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
    run = MSADecode(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0])
    run.scores.fill_(float("nan"))
    run.out.fill_(float("nan"))
    run(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
    torch.cuda.synchronize()
    return run


def _host_meta(dev):
    return dict(bt=host(dev.block_table), L=host(dev.ctx_len), pos=host(dev.q_pos), req=host(dev.q_req))


def _check_all_rows_decode(dev, run, m):
    wl = dev.wl
    s, sel, cnt = host(run.scores), host(run.sel), host(run.cnt)
    o_sel, o_cnt = oracle.topk_blocks(s.astype(np.float64), m["pos"], wl.block, wl.k)
    assert np.array_equal(sel, o_sel) and np.array_equal(cnt, o_cnt), "top-k differs on identical scores"
    ncand = m["pos"] // wl.block + 1
    assert np.all(cnt == np.minimum(wl.k, ncand)[:, None])
    pt, rl = host(run.page_table), host(run.row_len)
    o_pt, o_rl = oracle.sparse_page_table(sel, cnt, m["bt"], m["L"], m["req"], m["pos"], wl.Hkv, wl.block)
    assert np.array_equal(pt, o_pt) and np.array_equal(rl, o_rl)
    out = host(run.out)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(host(run.lse)))
    return s, sel, cnt, out


def _check_requests_decode(dev, run, m, reqs, s, sel, cnt, out, exact_hot=False):
    """Oracle on whole sampled requests (all KV heads, all candidate blocks)."""
    wl = dev.wl
    kidx, kc, vc = DeviceView(dev.kidx), DeviceView(dev.kcache), DeviceView(dev.vcache)
    lse = host(run.lse)
    for r in reqs:
        rows = np.nonzero(m["req"] == r)[0]
        qi = host(dev.q_idx[torch.from_numpy(rows).cuda()])
        ref_s = oracle.index_scores(qi, kidx, m["bt"], m["L"], m["req"][rows], m["pos"][rows], wl.block)
        got = s[rows]
        assert np.array_equal(np.isneginf(got), np.isneginf(ref_s))
        fin = np.isfinite(ref_s)
        assert np.abs(got[fin] - ref_s[fin]).max() <= 1e-2, f"request {r}: scores"
        r_sel, r_cnt = oracle.topk_blocks(ref_s, m["pos"][rows], wl.block, wl.k)
        selection_excused(sel[rows], cnt[rows], r_sel, r_cnt, ref_s, wl.k)
        q = host(dev.q[torch.from_numpy(rows).cuda()])
        ref_o, ref_l = oracle.sparse_attention(q, kc, vc, m["bt"], m["L"], m["req"][rows], m["pos"][rows],
                                               sel[rows], cnt[rows], wl.block, dev.scale)
        assert_attn_close(out[rows], ref_o, what=f"request {r} attention")
        assert np.abs(lse[rows] - ref_l).max() <= 1e-3
        for g in range(wl.Hkv):
            hb = dev.hot.get((int(r), g))
            if hb and exact_hot:
                assert sel[rows[0], g].tolist() == hb


def test_agentic_decode_full():
    wl = mi.agentic_decode()
    announce("full", wl.name)
    dev = mi.make_inputs(wl, "cuda")
    run = _decode_run(dev)
    m = _host_meta(dev)
    s, sel, cnt, out = _check_all_rows_decode(dev, run, m)
    _check_requests_decode(dev, run, m, [0, 5], s, sel, cnt, out, exact_hot=True)


@pytest.mark.parametrize("batch", [1, 4])
def test_million_decode_full(batch):
    wl = mi.million_decode(batch=batch)
    announce("full", wl.name)
    dev = mi.make_inputs(wl, "cuda")
    run = _decode_run(dev)
    m = _host_meta(dev)
    s, sel, cnt, out = _check_all_rows_decode(dev, run, m)
    # all 8192 blocks of every KV head of the last request (its rows sit past the others' pages)
    _check_requests_decode(dev, run, m, [batch - 1], s, sel, cnt, out)


def test_spec_decode_full():
    """Four query tokens per request share one pass of the scorer over each page."""
    wl = mi.spec_decode()
    announce("full", wl.name)
    dev = mi.make_inputs(wl, "cuda")
    run = _decode_run(dev)
    m = _host_meta(dev)
    s, sel, cnt, out = _check_all_rows_decode(dev, run, m)
    _check_requests_decode(dev, run, m, [0, 7], s, sel, cnt, out)


def test_ragged_decode_full():
    wl = mi.ragged_decode()
    announce("full", wl.name)
    dev = mi.make_inputs(wl, "cuda")
    run = _decode_run(dev)
    m = _host_meta(dev)
    s, sel, cnt, out = _check_all_rows_decode(dev, run, m)
    order = np.argsort(m["L"])
    reqs = [int(order[0]), int(order[len(order) // 2]), int(order[-1])]       # shortest, median, longest
    _check_requests_decode(dev, run, m, reqs, s, sel, cnt, out)


def test_long_prefill_full():
    msa = lib()
    from block_sparse_long_msa_amd.pipeline import MSAPrefill
    wl = mi.long_prefill()
    announce("full", wl.name)
    dev = mi.make_inputs(wl, "cuda")
    b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
    run = MSAPrefill(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0], fused=False)
    run.out.fill_(float("nan"))
    run(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
    torch.cuda.synchronize()
    m = _host_meta(dev)
    s, sel, cnt = host(run.scores), host(run.sel), host(run.cnt)
    # the fused scorer + top-k selects exactly the same blocks
    fused = MSAPrefill(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0], fused=True)
    fused(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
    assert np.array_equal(host(fused.sel), sel) and np.array_equal(host(fused.cnt), cnt)
    assert np.array_equal(host(fused.out).view(np.uint32), host(run.out).view(np.uint32))
    del fused
    # every row: exact top-k on the GPU's scores, counts, finite outputs, absent slots marked
    o_sel, o_cnt = oracle.topk_blocks(s.astype(np.float64), m["pos"], wl.block, wl.k)
    assert np.array_equal(sel, o_sel) and np.array_equal(cnt, o_cnt)
    out, lse, pl = host(run.out), host(run.lse), host(run.part_lse)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    present = np.arange(wl.k)[None, None, :] < cnt[:, :, None]
    assert np.all(np.isfinite(pl[present])) and np.all(np.isneginf(pl[~present]))
    # sampled rows: the request's caches on the host, the oracle row by row
    rows = np.linspace(0, wl.Nq - 1, 12).astype(int)
    kidx, kc, vc = host(dev.kidx), host(dev.kcache), host(dev.vcache)
    qi, q = host(dev.q_idx)[rows], host(dev.q)[rows]
    ref_s = oracle.index_scores(qi, kidx, m["bt"], m["L"], m["req"][rows], m["pos"][rows], wl.block)
    fin = np.isfinite(ref_s)
    assert np.array_equal(fin, np.isfinite(s[rows]))
    assert np.abs(s[rows][fin] - ref_s[fin]).max() <= 1e-2
    r_sel, r_cnt = oracle.topk_blocks(ref_s, m["pos"][rows], wl.block, wl.k)
    selection_excused(sel[rows], cnt[rows], r_sel, r_cnt, ref_s, wl.k)
    po = host(run.part_o)[rows]
    ref_po, ref_pl = oracle.block_partials(q, kc, vc, m["bt"], m["L"], m["req"][rows], m["pos"][rows], sel[rows],
                                           cnt[rows], wl.block, dev.scale)
    pr = present[rows]
    assert_attn_close(po[pr], ref_po[pr], what="sampled partials")
    assert np.abs(pl[rows][pr] - ref_pl[pr]).max() <= 1e-3
    ref_o, ref_l = oracle.sparse_attention(q, kc, vc, m["bt"], m["L"], m["req"][rows], m["pos"][rows], sel[rows],
                                           cnt[rows], wl.block, dev.scale)
    assert_attn_close(out[rows], ref_o, what="sampled merged output")
    assert np.abs(lse[rows] - ref_l).max() <= 1e-3
    # the query-major baseline selects the same blocks and gives the same attention on them
    from block_sparse_long_msa_amd.pipeline import MSAPrefillQueryMajor
    qm = MSAPrefillQueryMajor(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0])
    qm.out.fill_(float("nan"))
    qm(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
    torch.cuda.synchronize()
    assert np.array_equal(host(qm.sel), sel) and np.array_equal(host(qm.cnt), cnt)
    qo, ql = host(qm.out), host(qm.lse)
    assert np.all(np.isfinite(qo)) and np.all(np.isfinite(ql))
    assert_attn_close(qo[rows], ref_o, what="sampled query-major output")
    assert np.abs(ql[rows] - ref_l).max() <= 1e-3


def test_tiny_prefill_full():
    """The 2048-token workload is small enough for the oracle on every row."""
    msa = lib()
    from block_sparse_long_msa_amd.pipeline import MSAPrefill
    wl = mi.tiny_prefill()
    announce("full", wl.name)
    cpu = mi.make_inputs(wl, "cpu")
    dev = cpu.to("cuda")
    b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
    run = MSAPrefill(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0])
    run(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
    torch.cuda.synchronize()
    m = _host_meta(dev)
    sel, cnt = host(run.sel), host(run.cnt)
    f = lambda t: t.float().numpy()
    ref_s = oracle.index_scores(f(cpu.q_idx), f(cpu.kidx), m["bt"], m["L"], m["req"], m["pos"], wl.block)
    r_sel, r_cnt = oracle.topk_blocks(ref_s, m["pos"], wl.block, wl.k)
    selection_excused(sel, cnt, r_sel, r_cnt, ref_s, wl.k)
    for g in range(wl.Hkv):                       # the last token sees all four planted blocks
        assert sel[-1, g].tolist() == cpu.hot[(0, g)]
    ref_o, _ = oracle.sparse_attention(f(cpu.q), f(cpu.kcache), f(cpu.vcache), m["bt"], m["L"], m["req"], m["pos"],
                                       sel, cnt, wl.block, dev.scale)
    assert_attn_close(host(run.out), ref_o)
