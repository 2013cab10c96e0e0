"""Pins for the CPU oracle: brute force, closed forms, library special cases and invariants.

None of these re-types the oracle's own formula: scores are checked against pure-Python
per-token loops (math.fsum), closed forms and a hand-worked example; top-k against the
defining property over all subsets; attention against torch's scaled_dot_product_attention
(float64, CPU) with explicit masks; the merge against one softmax over the union; the page
table against torch.as_strided views of the flat cache.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _helpers import np_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(ctx, nq, block=16, Hq=4, Hkv=2, D=8, Di=3, k=3, seed=11, **kw):
    wl = mi.small_workload(ctx, nq, Hq=Hq, Hkv=Hkv, D=D, Di=Di, k=k, seed=seed, block=block, **kw)
    return np_inputs(mi.make_inputs(wl))


def _scores(x):
    return oracle.index_scores(x.q_idx, x.kidx, x.block_table, x.ctx_len, x.q_req, x.q_pos, x.wl.block)


def _select(x, k=None):
    s = _scores(x)
    sel, cnt = oracle.topk_blocks(s, x.q_pos, x.wl.block, k or x.wl.k)
    return s, sel, cnt


# --- hand-worked example --------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        return json.load(f)


def _golden_arrays(g):
    BS = g["block"]
    L = g["ctx_len"]
    bt = np.asarray([g["block_table"]], dtype=np.int32)
    P = max(g["block_table"]) + 1

    def cache(rows):
        c = np.zeros((P, BS, 1, 2))
        for s, row in enumerate(rows):
            c[bt[0, s // BS], s % BS, 0] = row
        return c
    return BS, L, bt, cache


def test_golden_scores_topk_pagetable():
    g = _golden()
    BS, L, bt, cache = _golden_arrays(g)
    kidx = cache(g["k_idx"])
    qi = np.asarray([[g["q_idx"]]])
    s = oracle.index_scores(qi, kidx, bt, np.asarray([L]), np.asarray([0]), np.asarray([g["q_pos"]]), BS)
    assert s[0, 0].tolist() == g["scores"]
    for k, key in ((1, "top1"), (2, "top2"), (5, "top5")):
        sel, cnt = oracle.topk_blocks(s, np.asarray([g["q_pos"]]), BS, k)
        assert sel[0, 0].tolist() == g[key]
    for k, key in ((2, "top2"), (5, "top5")):
        sel, cnt = oracle.topk_blocks(s, np.asarray([g["q_pos"]]), BS, k)
        pt, rl = oracle.sparse_page_table(sel, cnt, bt, np.asarray([L]), np.asarray([0]),
                                          np.asarray([g["q_pos"]]), 1, BS)
        assert pt[0].tolist() == g[f"page_table_{key}"]
        assert int(rl[0]) == g[f"row_len_{key}"]


@pytest.mark.parametrize("qkey,okey,lkey", [(None, "attention_q0_top2", "lse_q0_top2"),
                                            ("q_ln3", "attention_ln3_top2", "lse_ln3_top2")])
def test_golden_attention(qkey, okey, lkey):
    g = _golden()
    BS, L, bt, cache = _golden_arrays(g)
    K, V = cache(g["k"]), cache(g["v"])
    q = np.zeros((1, 1, 2)) if qkey is None else np.asarray([[g[qkey]]])
    sel = np.asarray([[[0, 1]]], dtype=np.int32)
    cnt = np.asarray([[2]], dtype=np.int32)
    out, lse = oracle.sparse_attention(q, K, V, bt, np.asarray([L]), np.asarray([0]), np.asarray([g["q_pos"]]),
                                       sel, cnt, BS, 1.0 / math.sqrt(2.0))
    np.testing.assert_allclose(out[0, 0], g[okey], rtol=0, atol=1e-12)
    assert abs(lse[0, 0] - g[lkey]) < 1e-12
    po, pl = oracle.block_partials(q, K, V, bt, np.asarray([L]), np.asarray([0]), np.asarray([g["q_pos"]]),
                                   sel, cnt, BS, 1.0 / math.sqrt(2.0))
    o2, l2 = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(o2[0, 0, 0], g[okey], rtol=0, atol=1e-12)
    assert abs(l2[0, 0, 0] - g[lkey]) < 1e-12


# --- scores -------------------------------------------------------------------------

def _bruteforce_scores(x):
    """Per-token Python loops with math.fsum; a block's score is the max over its valid tokens."""
    BS = x.wl.block
    Nq, Hkv, Di = x.q_idx.shape
    out = np.full((Nq, Hkv, x.block_table.shape[1]), -np.inf)
    for t in range(Nq):
        r, p = int(x.q_req[t]), int(x.q_pos[t])
        L = int(x.ctx_len[r])
        for g in range(Hkv):
            for s in range(L):
                if s > p:
                    continue
                page = int(x.block_table[r, s // BS])
                dot = math.fsum(float(x.q_idx[t, g, d]) * float(x.kidx[page, s % BS, g, d]) for d in range(Di))
                b = s // BS
                out[t, g, b] = max(out[t, g, b], dot)
    return out


@pytest.mark.parametrize("ctx,nq,seed", [([37, 70], [5, 3], 1), ([16, 17, 1], [16, 2, 1], 2), ([100], [100], 3)])
def test_scores_bruteforce(ctx, nq, seed):
    x = _tiny(ctx, nq, seed=seed)
    ref = _bruteforce_scores(x)
    got = _scores(x)
    assert np.array_equal(np.isneginf(ref), np.isneginf(got))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=0, atol=1e-11)


def test_scores_identical_rows_closed_form():
    x = _tiny([64], [1], Di=5, seed=4)
    page = int(x.block_table[0, 1])
    row = np.array([0.5, -1.25, 2.0, 0.75, -0.5])
    x.kidx[page, :, 1, :] = row
    s = _scores(x)
    expect = float(np.dot(x.q_idx[0, 1].astype(np.float64), row))
    assert s[0, 1, 1] == pytest.approx(expect, abs=1e-12)


def test_scores_one_dim_closed_form():
    x = _tiny([90], [3], Di=1, seed=5)
    s = _scores(x)
    BS = x.wl.block
    for t in range(3):
        p = int(x.q_pos[t])
        for g in range(2):
            qv = float(x.q_idx[t, g, 0])
            for b in range(p // BS + 1):
                ks = [float(x.kidx[int(x.block_table[0, b]), i, g, 0]) for i in range(BS) if b * BS + i <= p]
                assert s[t, g, b] == pytest.approx(qv * (max(ks) if qv >= 0 else min(ks)), abs=1e-12)
            assert np.all(np.isneginf(s[t, g, p // BS + 1:]))


# --- top-k -------------------------------------------------------------------------------

def _topk_by_definition(s, k):
    """The unique subset S, |S| = min(k, n), such that each member beats each non-member
    under (score desc, id asc)."""
    n = len(s)
    beats = lambda a, b: s[a] > s[b] or (s[a] == s[b] and a < b)
    hits = [c for c in itertools.combinations(range(n), min(k, n))
            if all(beats(a, b) for a in c for b in range(n) if b not in c)]
    assert len(hits) == 1
    return list(hits[0])


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(0)
    BS = 4
    for trial in range(300):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 11))
        vals = rng.integers(-3, 3, size=n).astype(np.float64)     # many exact ties
        scores = np.full((1, 1, 12), -np.inf)
        scores[0, 0, :n] = vals
        pos = np.asarray([(n - 1) * BS + int(rng.integers(0, BS))])
        sel, cnt = oracle.topk_blocks(scores, pos, BS, k)
        want = _topk_by_definition(vals, k)
        assert cnt[0, 0] == len(want)
        assert sel[0, 0, :cnt[0, 0]].tolist() == want            # ascending
        assert np.all(sel[0, 0, cnt[0, 0]:] == -1)


def test_topk_all_when_few_candidates():
    x = _tiny([40], [40], k=8, seed=6)
    _, sel, cnt = _select(x)
    for t in range(40):
        n = int(x.q_pos[t]) // x.wl.block + 1
        assert np.all(cnt[t] == n)
        assert np.all(sel[t, :, :n] == np.arange(n)) and np.all(sel[t, :, n:] == -1)


def test_topk_invariant_to_positive_scaling():
    x = _tiny([300, 129], [4, 2], Di=16, k=3, seed=7)
    s1, sel1, cnt1 = _select(x)
    x.q_idx = x.q_idx * 2.0          # exact in binary floating point
    s2, sel2, cnt2 = _select(x)
    assert np.array_equal(sel1, sel2) and np.array_equal(cnt1, cnt2)
    fin = np.isfinite(s1)
    np.testing.assert_allclose(s2[fin], 2.0 * s1[fin], rtol=1e-12)


def test_topk_invariant_to_page_permutation():
    x = _tiny([300, 129], [4, 2], Di=16, k=3, seed=8)
    s1, sel1, cnt1 = _select(x)
    P = x.kidx.shape[0]
    perm = np.random.default_rng(1).permutation(P)
    kidx2 = np.empty_like(x.kidx)
    kidx2[perm] = x.kidx
    x.kidx = kidx2
    x.block_table = perm[x.block_table].astype(np.int32)
    s2, sel2, cnt2 = _select(x)
    assert np.array_equal(s1, s2) and np.array_equal(sel1, sel2)


def test_topk_finds_planted_hot_blocks():
    wl = mi.small_workload([4000, 2500], [1, 1], Hq=8, Hkv=2, D=64, Di=128, k=6, seed=9,
                           hot_per_group=6, hot_ref="query")
    x = np_inputs(mi.make_inputs(wl))
    _, sel, cnt = _select(x)
    for (r, g), hb in x.hot.items():
        assert sel[r, g].tolist() == hb


# --- attention ------------------------------------------------------------------------------------

def _sdpa(qh, K, V, mask, scale):
    """torch SDPA in float64 on the CPU for one head: qh [T, D], K/V [S, D], mask [T, S] bool."""
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qh)[None, None], torch.from_numpy(K)[None, None], torch.from_numpy(V)[None, None],
        attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    return o[0, 0].numpy()


def _attend(x, sel, cnt):
    return oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                   sel, cnt, x.wl.block, x.scale)


@pytest.mark.parametrize("ctx,nq", [([70], [70]), ([130, 45], [9, 45])])
def test_attention_all_blocks_equals_dense_causal_gqa(ctx, nq):
    x = _tiny(ctx, nq, k=64, D=8, seed=12)
    _, sel, cnt = _select(x)
    out, _ = _attend(x, sel, cnt)
    G = x.wl.G
    for r, L in enumerate(ctx):
        rows = np.nonzero(x.q_req == r)[0]
        K = oracle.request_tokens(x.kcache, x.block_table[r], L, x.wl.block)
        V = oracle.request_tokens(x.vcache, x.block_table[r], L, x.wl.block)
        mask = np.arange(L)[None, :] <= x.q_pos[rows][:, None]
        for h in range(x.wl.Hq):
            ref = _sdpa(x.q[rows, h].astype(np.float64), K[:, h // G], V[:, h // G], mask, x.scale)
            np.testing.assert_allclose(out[rows, h], ref, rtol=0, atol=1e-12)


def test_attention_equals_block_masked_sdpa():
    x = _tiny([200], [60], k=3, D=8, Di=4, seed=13)
    _, sel, cnt = _select(x)
    out, _ = _attend(x, sel, cnt)
    BS, L, G = x.wl.block, 200, x.wl.G
    K = oracle.request_tokens(x.kcache, x.block_table[0], L, BS)
    V = oracle.request_tokens(x.vcache, x.block_table[0], L, BS)
    for g in range(x.wl.Hkv):
        blk = np.arange(L) // BS
        chosen = np.zeros((60, L), dtype=bool)
        for t in range(60):
            chosen[t] = np.isin(blk, sel[t, g, :cnt[t, g]])
        mask = chosen & (np.arange(L)[None, :] <= x.q_pos[:, None])
        for h in range(g * G, (g + 1) * G):
            ref = _sdpa(x.q[:, h].astype(np.float64), K[:, g], V[:, g], mask, x.scale)
            np.testing.assert_allclose(out[:, h], ref, rtol=0, atol=1e-12)


def test_attention_zero_query_is_mean_of_selected_values():
    x = _tiny([150, 77], [3, 2], k=2, D=8, seed=14)
    _, sel, cnt = _select(x)
    x.q = np.zeros_like(x.q)
    out, lse = _attend(x, sel, cnt)
    BS = x.wl.block
    for t in range(5):
        r, p = int(x.q_req[t]), int(x.q_pos[t])
        for h in range(x.wl.Hq):
            g = h // x.wl.G
            rows = [x.vcache[int(x.block_table[r, b]), s, g].astype(np.float64)
                    for b in sel[t, g, :cnt[t, g]] for s in range(BS)
                    if b * BS + s <= p and b * BS + s < x.ctx_len[r]]
            np.testing.assert_allclose(out[t, h], np.mean(rows, axis=0), atol=1e-12)
            assert lse[t, h] == pytest.approx(math.log(len(rows)), abs=1e-12)


# --- LSE merge ------------------------------------------------------------------------------

def test_merged_partials_equal_one_softmax_over_union():
    x = _tiny([300, 90], [20, 7], k=3, D=8, Di=4, seed=15)
    _, sel, cnt = _select(x)
    out, lse = _attend(x, sel, cnt)
    po, pl = oracle.block_partials(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                   sel, cnt, x.wl.block, x.scale)
    o2, l2 = oracle.lse_merge(po, pl)
    Nq, Hq, D = out.shape
    np.testing.assert_allclose(o2.reshape(Nq, Hq, D), out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2.reshape(Nq, Hq), lse, rtol=0, atol=1e-12)


def test_merge_single_part_and_equal_lse():
    rng = np.random.default_rng(3)
    po = rng.normal(size=(4, 1, 2, 5))
    pl = rng.normal(size=(4, 1, 2))
    o, l = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(o, po[:, 0], atol=1e-14)
    np.testing.assert_allclose(l, pl[:, 0], atol=1e-14)
    po = rng.normal(size=(3, 4, 2, 5))
    pl = np.full((3, 4, 2), 0.7)
    o, l = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(o, po.mean(axis=1), atol=1e-14)
    np.testing.assert_allclose(l, 0.7 + math.log(4), atol=1e-14)
    pl[:, 1:] = -np.inf
    po[:, 1:] = np.nan               # empty slots are never read
    o, l = oracle.lse_merge(po, pl)
    np.testing.assert_allclose(o, po[:, 0], atol=1e-14)


# --- decode page table over strided views ------------------------------------------------------

def test_page_table_addresses_round_trip_through_as_strided():
    x = _tiny([300, 47, 129], [1, 1, 1], k=3, D=8, seed=16)
    _, sel, cnt = _select(x)
    Hkv, BS, D = x.wl.Hkv, x.wl.block, x.wl.D
    pt, rl = oracle.sparse_page_table(sel, cnt, x.block_table, x.ctx_len, x.q_req, x.q_pos, Hkv, BS)
    flat = torch.from_numpy(x.kcache).reshape(-1)
    for t in range(3):
        for g in range(Hkv):
            for j in range(cnt[t, g]):
                v = int(pt[t * Hkv + g, j])
                view = torch.as_strided(flat, (BS, D), (Hkv * D, 1), storage_offset=v * D)
                page = int(x.block_table[int(x.q_req[t]), sel[t, g, j]])
                assert torch.equal(view, torch.from_numpy(x.kcache[page, :, g, :]))
            L = int(x.ctx_len[t])
            full = cnt[t, g] * BS
            last_sel = int(sel[t, g, cnt[t, g] - 1])
            expect = full - (BS - (L - last_sel * BS)) if last_sel == (L - 1) // BS else full
            assert rl[t * Hkv + g] == expect


def test_paged_decode_attention_equals_block_table_attention():
    x = _tiny([300, 47, 129, 256], [1, 1, 1, 1], Hq=8, Hkv=2, k=3, D=8, seed=17)
    _, sel, cnt = _select(x)
    out, lse = _attend(x, sel, cnt)
    Hkv, BS, D, G = x.wl.Hkv, x.wl.block, x.wl.D, x.wl.G
    pt, rl = oracle.sparse_page_table(sel, cnt, x.block_table, x.ctx_len, x.q_req, x.q_pos, Hkv, BS)
    q_rows = x.q.reshape(4 * Hkv, G, D)
    o2, l2 = oracle.paged_decode_attention(q_rows, x.kcache, x.vcache, pt, rl, D, Hkv * D, BS, x.scale)
    np.testing.assert_allclose(o2.reshape(out.shape), out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2.reshape(lse.shape), lse, rtol=0, atol=1e-12)


def test_decode_equals_last_prefill_token():
    """One query at pos = L - 1 (decode: page table over strided views, one attention per row)
    gives what the prefill of the whole context gives for its last token (KV-block-major lists,
    per-block partials, LSE merge): the two routes share only the score and selection steps."""
    x = _tiny([203], [203], Hq=4, Hkv=2, D=8, k=4, seed=19)
    Nq, Hkv, G, D, BS = 203, x.wl.Hkv, x.wl.G, x.wl.D, x.wl.block
    _, sel, cnt = _select(x)
    po, pl = oracle.block_partials(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                   sel, cnt, BS, x.scale)
    o_pre, l_pre = oracle.lse_merge(po, pl)                       # [Nq, Hkv, G, D], [Nq, Hkv, G]
    last = slice(Nq - 1, Nq)
    assert int(x.q_pos[-1]) == int(x.ctx_len[0]) - 1
    s_dec = oracle.index_scores(x.q_idx[last], x.kidx, x.block_table, x.ctx_len, x.q_req[last], x.q_pos[last], BS)
    sel_d, cnt_d = oracle.topk_blocks(s_dec, x.q_pos[last], BS, x.wl.k)
    pt, rl = oracle.sparse_page_table(sel_d, cnt_d, x.block_table, x.ctx_len, x.q_req[last], x.q_pos[last], Hkv, BS)
    o_dec, l_dec = oracle.paged_decode_attention(x.q[last].reshape(Hkv, G, D), x.kcache, x.vcache, pt, rl, D,
                                                 Hkv * D, BS, x.scale)
    assert np.array_equal(sel_d[0], sel[-1]) and np.array_equal(cnt_d[0], cnt[-1])
    np.testing.assert_allclose(o_dec, o_pre[-1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_dec, l_pre[-1], rtol=0, atol=1e-12)


def test_kv_block_major_lists_invert_the_selection():
    x = _tiny([300], [50], k=3, seed=18)
    _, sel, cnt = _select(x)
    lists = oracle.kv_block_major_lists(sel, cnt, x.block_table, x.q_req, x.wl.Hkv)
    assert sum(len(v) for v in lists.values()) == int(cnt.sum())
    for (g, p), entries in lists.items():
        for t, j in entries:
            assert int(x.block_table[0, sel[t, g, j]]) == p


# --- the pins catch planted mistakes ------------------------------------------------------------

def test_pins_catch_off_by_one_causal_mask(monkeypatch):
    x = _tiny([37, 70], [5, 3], seed=1)
    ref = _bruteforce_scores(x)
    orig = oracle.msa_oracle.valid_token_count
    monkeypatch.setattr(oracle.msa_oracle, "valid_token_count",
                        lambda b, pos, L, block: orig(b, pos + 1, L, block))
    got = _scores(x)
    fin = np.isfinite(ref)
    assert not np.allclose(got[fin], ref[fin], atol=1e-11)


def test_pins_catch_missing_softmax_scale(monkeypatch):
    x = _tiny([70], [70], k=64, D=8, seed=12)
    _, sel, cnt = _select(x)
    x.scale = 1.0                    # the planted mistake: logits unscaled in the oracle call
    out, _ = _attend(x, sel, cnt)
    K = oracle.request_tokens(x.kcache, x.block_table[0], 70, x.wl.block)
    V = oracle.request_tokens(x.vcache, x.block_table[0], 70, x.wl.block)
    mask = np.arange(70)[None, :] <= x.q_pos[:, None]
    ref = _sdpa(x.q[:, 0].astype(np.float64), K[:, 0], V[:, 0], mask, 1.0 / math.sqrt(8))
    assert not np.allclose(out[:, 0], ref, atol=1e-6)


def test_pins_catch_reversed_tie_rule(monkeypatch):
    """A top-k that prefers the higher block id among equal scores fails the defining property."""
    orig = np.lexsort

    def lexsort_higher_id_first(keys):
        ids, neg_s = keys
        return orig((-np.asarray(ids), neg_s))
    monkeypatch.setattr(oracle.msa_oracle.np, "lexsort", lexsort_higher_id_first)
    vals = np.asarray([1.0, 2.0, 1.0, 1.0, 0.0])          # three-way tie at the boundary for k = 2
    scores = np.full((1, 1, 8), -np.inf)
    scores[0, 0, :5] = vals
    sel, cnt = oracle.topk_blocks(scores, np.asarray([4 * 4]), 4, 2)
    assert sel[0, 0, :cnt[0, 0]].tolist() != _topk_by_definition(vals, 2)


def test_pins_catch_base2_lse(monkeypatch):
    """A merge that takes log2 of the weight sum no longer equals one softmax over the union."""
    monkeypatch.setattr(oracle.msa_oracle.np, "log", np.log2)
    x = _tiny([300, 90], [20, 7], k=3, D=8, Di=4, seed=15)
    _, sel, cnt = _select(x)
    po, pl = oracle.block_partials(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                   sel, cnt, x.wl.block, x.scale)
    _, l2 = oracle.lse_merge(po, pl)
    monkeypatch.undo()
    _, lse = _attend(x, sel, cnt)
    assert not np.allclose(l2.reshape(lse.shape), lse, atol=1e-6)


def test_pins_catch_mean_block_score(monkeypatch):
    """Reducing a block by the mean of its tokens' dots instead of the max fails the brute force."""
    monkeypatch.setattr(oracle.msa_oracle, "block_score",
                        lambda q_vec, k_rows, n_valid: float(np.mean(k_rows[:n_valid] @ q_vec)))
    x = _tiny([37, 70], [5, 3], seed=1)
    got = _scores(x)
    monkeypatch.undo()
    ref = _bruteforce_scores(x)
    fin = np.isfinite(ref)
    assert not np.allclose(got[fin], ref[fin], atol=1e-9)


def test_pins_catch_page_id_without_head_stride():
    """A virtual page id of block_table*block + g (forgetting the factor Hkv) addresses other rows:
    the as_strided round trip pin fails on it."""
    x = _tiny([300, 47], [1, 1], k=3, D=8, seed=16)
    _, sel, cnt = _select(x)
    Hkv, BS, D = x.wl.Hkv, x.wl.block, x.wl.D
    flat = torch.from_numpy(x.kcache).reshape(-1)
    mismatches = 0
    for t in range(2):
        for g in range(Hkv):
            for j in range(cnt[t, g]):
                page = int(x.block_table[int(x.q_req[t]), sel[t, g, j]])
                v = page * BS + g                                  # the planted mistake
                view = torch.as_strided(flat, (BS, D), (Hkv * D, 1), storage_offset=v * D)
                mismatches += not torch.equal(view, torch.from_numpy(x.kcache[page, :, g, :]))
    assert mismatches > 0
