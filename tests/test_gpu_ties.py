"""The top-k tie rule at the k-th boundary, checked strictly against the oracle on every top-k route.

Each request and KV group has its own top-k boundary (Chinese page, section "索引评分器成为解码关键路径"),
and selections may legitimately differ only at near-ties there (SGLang M3.1 post, "Miles Day-0
Support"); the library fixes the rule: equal scores prefer the lower block id.  For every decode row
this test copies the key-index rows of the row's k-th best block bitwise into one of its unselected
full blocks, so the two blocks score exactly the same on both sides (same bytes, same arithmetic).
Half the rows get the copy at a lower block id (which must then replace the k-th block), half at a
higher one (which must stay out).  The selections of msa_topk_blocks, msa_topk_page_table and
msa_topk_attn_decode must then equal the oracle's top-k on the oracle's own fp64 scores, with no
boundary excusal.  Context lengths walk through the register layouts of the top-k (one wave with
1, 4 and 8 scores per lane; 4 and 16 waves with 8 and 16 scores per lane, which select in two levels,
so a copy often lands in another wave's run of ids than the block it ties) and the radix select beyond
16,384 blocks.
"""
import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _gpu import announce, batch, host, scores, setup, topk, topk_attn_decode, topk_page_table

pytestmark = pytest.mark.gpu

CASES = {  # name: (context lengths, Hkv, k)
    "one_wave_1_per_lane": ([5000, 7001, 3333], 2, 8),
    "one_wave_4_per_lane": ([30000, 25000], 2, 16),
    "one_wave_8_per_lane": ([60000, 50001], 2, 16),
    "four_waves": ([140000, 190000], 2, 33),
    "four_waves_16_per_lane": ([300000, 400000], 2, 24),
    "sixteen_waves": ([524300], 1, 32),
    "sixteen_waves_16_per_lane": ([1500000], 1, 48),
    "radix_select": ([2100000], 1, 9),
}
GPU_DRAWN = {"sixteen_waves", "sixteen_waves_16_per_lane", "radix_select"}


def _order(row, n):
    """Candidate ids of one score row by (score desc, id asc)."""
    ids = np.arange(n)
    return np.lexsort((ids, -row[:n]))


def _plant_ties(dev, s, k):
    """Copy the k-th block's key-index rows into an unselected full block of every (row, KV head)
    that has one; returns {(t, g): (kth_block, copy_block)}."""
    wl = dev.wl
    bt, pos = host(dev.block_table), host(dev.q_pos)
    planted = {}
    for t in range(wl.Nq):           # one query per request: row t is request t
        n = int(pos[t]) // wl.block + 1
        full = (int(pos[t]) + 1) // wl.block          # blocks 0 .. full-1 have every token valid
        for g in range(wl.Hkv):
            order = _order(s[t, g], n)
            if n <= k:
                continue
            kth = int(order[k - 1])
            if kth >= full:
                continue
            rest = np.sort(order[k:][order[k:] < full])
            want_lower = (t + g) % 2 == 0
            cand = rest[rest < kth] if want_lower else rest[rest > kth]
            if len(cand) == 0:
                continue
            dst = int(cand[len(cand) // 2])
            src_page, dst_page = int(bt[t, kth]), int(bt[t, dst])
            dev.kidx[dst_page, :, g, :] = dev.kidx[src_page, :, g, :]
            planted[(t, g)] = (kth, dst)
    return planted


@pytest.mark.parametrize("name", list(CASES))
def test_boundary_ties_follow_the_lower_id_rule(name):
    ctx, Hkv, k = CASES[name]
    announce("boundary ties", name)
    wl = mi.small_workload(ctx, [1] * len(ctx), Hq=4 * Hkv, Hkv=Hkv, D=64, Di=64, k=k, seed=77)
    dev, _ = setup(wl, on_gpu_generation=name in GPU_DRAWN)
    b = batch(dev)
    planted = _plant_ties(dev, host(scores(dev, b)), k)
    assert len(planted) >= max(1, wl.Nq * Hkv // 2), f"too few ties planted: {len(planted)}"
    torch.cuda.synchronize()

    s = scores(dev, b)                               # the caches now hold the copies
    sg = host(s)
    cpu = dev.to("cpu")
    f = lambda t: t.float().numpy()
    i = lambda t: t.numpy()
    ref = oracle.index_scores(f(cpu.q_idx), f(cpu.kidx), i(cpu.block_table), i(cpu.ctx_len), i(cpu.q_req),
                              i(cpu.q_pos), wl.block)
    for (t, g), (kth, dst) in planted.items():
        assert ref[t, g, kth] == ref[t, g, dst], "the oracle's scores of the copied blocks differ"
        assert sg[t, g, kth] == sg[t, g, dst], "the GPU's scores of the copied blocks differ"
        n = int(i(cpu.q_pos)[t]) // wl.block + 1
        order = _order(ref[t, g], n)
        assert ref[t, g, order[k - 1]] == ref[t, g, order[k]], "the planted tie is not at the k-th boundary"
    o_sel, o_cnt = oracle.topk_blocks(ref, i(cpu.q_pos), wl.block, k)
    for (t, g), (kth, dst) in planted.items():     # the rule as stated, on the oracle's side
        chosen = set(o_sel[t, g, :o_cnt[t, g]].tolist())
        assert min(kth, dst) in chosen and max(kth, dst) not in chosen

    routes = {"msa_topk_blocks": topk(dev, b, s), "msa_topk_page_table": topk_page_table(dev, b, s)[:2],
              "msa_topk_attn_decode": topk_attn_decode(dev, b, s)[:2]}
    for route, (sel, cnt) in routes.items():
        assert np.array_equal(host(sel), o_sel) and np.array_equal(host(cnt), o_cnt), f"{route}: tie rule broken"
