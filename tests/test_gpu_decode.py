"""GPU parity of the decode path (scorer, top-k, page table, decode attention, merge) against the
CPU oracle on identical seeded inputs, at sizes the oracle finishes in seconds.

Bars: scores |gpu - oracle| <= 1e-2; top-k bit-exact against the oracle run on the GPU's own
fp32 scores, and equal to the oracle's selection except at the k-th boundary (oracle scores
within 1e-3); page table bit-exact; attention |gpu - oracle| <= 2e-2 + 1e-2*|oracle| (bf16
output against the fp64 oracle) on identical selections, LSE within 1e-3.
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _gpu import (announce, batch, decode_attention, host, lib, page_table, scores, setup, topk, topk_attn_decode,
                  topk_page_table)
from _helpers import assert_attn_close, np_inputs, selection_excused

pytestmark = pytest.mark.gpu

CASES = {
    "edge_lengths_d64": dict(ctx=[300, 129, 1000, 128, 1, 127, 256, 257], nq=[1] * 8, Hq=8, Hkv=2, D=64, Di=64, k=4),
    "gqa8_d128_hot": dict(ctx=[5000, 2049, 777, 12345], nq=[1] * 4, Hq=64, Hkv=8, D=128, Di=128, k=16,
                          hot_per_group=16),
    "multi_query": dict(ctx=[4000, 300, 2000], nq=[3, 16, 8], Hq=16, Hkv=2, D=128, Di=128, k=8),
    "k_exceeds_candidates": dict(ctx=[500, 200, 129], nq=[1, 1, 1], Hq=8, Hkv=2, D=128, Di=64, k=16),
    "g16_d64_di128": dict(ctx=[3000, 1500], nq=[2, 1], Hq=32, Hkv=2, D=64, Di=128, k=5),
    "g1_d128": dict(ctx=[1800, 900], nq=[1, 1], Hq=4, Hkv=4, D=128, Di=128, k=3),
    # Hkv * Di > 1024: the decode scorer's direct-to-register variant
    "hkv16_direct_scorer": dict(ctx=[900, 400], nq=[1, 2], Hq=32, Hkv=16, D=64, Di=128, k=3),
    # few long rows: the register top-k holds a row in 16 waves (> 4096 blocks) or 4 waves (> 1024)
    "topk_16_waves": dict(ctx=[524300, 300001], nq=[1, 1], Hq=4, Hkv=1, D=64, Di=64, k=20),
    # 16 waves with 16 scores per lane (8193 to 16384 blocks): the two-level selection
    "topk_16_waves_two_level": dict(ctx=[1500000, 1100000], nq=[1, 1], Hq=4, Hkv=1, D=64, Di=64, k=40),
    # its edges: 8193 blocks (the last wave holds one candidate) and the largest k; a wave run of ids
    # ends exactly at the second row's last block
    "topk_two_level_edges": dict(ctx=[1048577, 1179648], nq=[1, 1], Hq=4, Hkv=1, D=64, Di=64, k=64),
    "topk_4_waves": dict(ctx=[190000, 140000], nq=[1, 1], Hq=8, Hkv=2, D=64, Di=64, k=33),
    # one wave holding 4 and 8 scores per lane (up to 256 / 512 blocks)
    "topk_4_per_lane": dict(ctx=[30000, 700], nq=[1, 2], Hq=8, Hkv=2, D=64, Di=64, k=7),
    "topk_8_per_lane": dict(ctx=[60000, 33000], nq=[1, 1], Hq=8, Hkv=2, D=64, Di=64, k=64),
    # >= 4096 rows of short candidate lists
    "many_rows": dict(ctx=[3000] * 2 + [700] * 254, nq=[1] * 256, Hq=32, Hkv=16, D=64, Di=64, k=6),
    # rows beyond the register layouts (> 16384 blocks): the radix-pass top-k, 16 waves per row,
    # and the two-launch form of msa_topk_page_table
    "topk_radix_long_rows": dict(ctx=[2100000], nq=[1], Hq=4, Hkv=1, D=64, Di=64, k=9),
    # the largest k and G: a row split into up to 64 page runs, merged over 64 parts
    "k64_g16_split": dict(ctx=[9000, 8300], nq=[1, 1], Hq=32, Hkv=2, D=128, Di=64, k=64),
    # the most KV heads the library takes (64, one query head each) with the largest k
    "hkv64_g1_k64": dict(ctx=[9000, 700], nq=[1, 2], Hq=64, Hkv=64, D=64, Di=64, k=64),
}
GPU_DRAWN = {"topk_16_waves", "topk_16_waves_two_level", "topk_two_level_edges", "topk_radix_long_rows"}   # inputs drawn on the GPU, copied to the host


def _wl(name, seed=21):
    c = dict(CASES[name])
    ctx, nq = c.pop("ctx"), c.pop("nq")
    return mi.small_workload(ctx, nq, seed=seed, **c)


def _run(dev, max_q=None):
    b = batch(dev, max_q)
    s = scores(dev, b)
    sel, cnt = topk(dev, b, s)
    pt, rl = page_table(dev, b, sel, cnt)
    # the one-call form gives the same four arrays bit for bit
    for a, f in zip((sel, cnt, pt, rl), topk_page_table(dev, b, s)):
        assert torch.equal(a, f), "msa_topk_page_table differs from msa_topk_blocks + msa_build_sparse_page_table"
    out, lse = decode_attention(dev, pt, rl)
    # top-k, page table and attention in one call: the same six arrays bit for bit
    for a, f in zip((sel, cnt, pt, rl, out, lse), topk_attn_decode(dev, b, s)):
        assert torch.equal(a, f), "msa_topk_attn_decode differs from the separate calls"
    return s, sel, cnt, pt, rl, out, lse


@pytest.mark.parametrize("name", list(CASES))
def test_decode_path_matches_oracle(name):
    announce("decode", name)
    dev, cpu = setup(_wl(name), on_gpu_generation=name in GPU_DRAWN, host_copy=True)
    _check_against_oracle(dev, cpu)


def test_queries_before_the_context_end():
    """Queries placed well before their request's last cached token: the blocks after every query's
    position but inside the context are streamed by the decode scorer with all of their tokens
    masked, so they must come out -inf, and attention stops at each query's own position."""
    announce("decode", "queries before the context end")
    dev, cpu = setup(_wl("multi_query", seed=9))
    pos, cu = cpu.q_pos.clone(), cpu.cu_q.numpy()
    for r, back in enumerate((2200, 0, 901)):     # contexts 4000, 300, 2000
        pos[cu[r]:cu[r + 1]] -= back
    cpu.q_pos, dev.q_pos = pos, pos.cuda()
    _check_against_oracle(dev, cpu)


def _check_against_oracle(dev, cpu):
    x = np_inputs(cpu)
    wl = dev.wl
    s, sel, cnt, pt, rl, out, lse = [host(t) for t in _run(dev)]

    ref_s = oracle.index_scores(x.q_idx, x.kidx, x.block_table, x.ctx_len, x.q_req, x.q_pos, wl.block)
    assert np.array_equal(np.isneginf(s), np.isneginf(ref_s)), "candidate masks differ"
    fin = np.isfinite(ref_s)
    assert np.abs(s[fin] - ref_s[fin]).max() <= 1e-2

    o_sel, o_cnt = oracle.topk_blocks(s.astype(np.float64), x.q_pos, wl.block, wl.k)
    assert np.array_equal(sel, o_sel) and np.array_equal(cnt, o_cnt), "top-k differs on identical scores"
    r_sel, r_cnt = oracle.topk_blocks(ref_s, x.q_pos, wl.block, wl.k)
    selection_excused(sel, cnt, r_sel, r_cnt, ref_s, wl.k)
    # planted hot blocks are biased toward the request's last query, which must choose them all (k permitting)
    if wl.hot_ref == "query":
        for (r, g), hb in x.hot.items():
            t_last = int(x.cu_q[r + 1]) - 1
            if len(hb) <= wl.k and t_last >= int(x.cu_q[r]):
                assert set(hb) <= set(sel[t_last, g, :cnt[t_last, g]].tolist()), f"request {r} group {g}: hot blocks"

    o_pt, o_rl = oracle.sparse_page_table(sel, cnt, x.block_table, x.ctx_len, x.q_req, x.q_pos, wl.Hkv, wl.block)
    assert np.array_equal(pt, o_pt) and np.array_equal(rl, o_rl)

    ref_o, ref_l = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, wl.block, x.scale)
    assert_attn_close(out, ref_o)
    assert np.abs(lse - ref_l).max() <= 1e-3


def test_decode_shapes_through_the_prefill_scorer():
    """The same decode rows scored by the GEMM kernel (hint > 16 queries per request)."""
    announce("decode rows via prefill scorer")
    dev, cpu = setup(_wl("gqa8_d128_hot"))
    x = np_inputs(cpu)
    s = host(scores(dev, batch(dev, max_q=64)))
    ref_s = oracle.index_scores(x.q_idx, x.kidx, x.block_table, x.ctx_len, x.q_req, x.q_pos, 128)
    assert np.array_equal(np.isneginf(s), np.isneginf(ref_s))
    fin = np.isfinite(ref_s)
    assert np.abs(s[fin] - ref_s[fin]).max() <= 1e-2


def test_decode_is_deterministic():
    announce("decode determinism")
    dev, _ = setup(_wl("gqa8_d128_hot", seed=5))
    a = [host(t) for t in _run(dev)]
    b = [host(t) for t in _run(dev)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_merge_matches_oracle():
    announce("lse merge")
    msa = lib()
    for rows, parts, G, D, seed in ((37, 16, 8, 128, 1), (5, 1, 4, 64, 2), (64, 7, 16, 64, 3), (9, 64, 1, 128, 4)):
        po, pl = mi.random_partials(rows, parts, G, D, seed)
        out = torch.full((rows, G, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((rows, G), float("nan"), device="cuda")
        msa.msa_lse_merge(rows, parts, G, D, po.cuda(), pl.cuda(), out, lse)
        ref_o, ref_l = oracle.lse_merge(po.float().numpy(), pl.numpy())
        assert_attn_close(host(out), ref_o, what=f"merge {rows}x{parts}x{G}x{D}")
        assert np.abs(host(lse) - ref_l).max() <= 1e-4
