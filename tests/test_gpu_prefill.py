"""GPU parity of the prefill path (GEMM scorer, top-k, remap + KV-block-major attention, LSE merge)
against the CPU oracle on identical seeded inputs.

Bars as for decode; the per-block partials (bf16) are compared slot by slot with the oracle's
block_partials on the GPU's selection, and the merged output with the oracle's one softmax over
the union of the selected blocks.
"""
import numpy as np
import pytest

import msa_inputs as mi
import oracle
from _gpu import announce, batch, decode_attention, host, lib, poison_i32, prefill, scores, setup, topk, topk_page_table
from _helpers import assert_attn_close, check_slot_of, expected_partials, np_inputs, selection_excused

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_prefill_2k": None,   # the 2048-token workload itself
    "ragged_multi_request": dict(ctx=[700, 300, 1000], nq=[300, 300, 129], Hq=16, Hkv=2, D=128, Di=128, k=5),
    "chunk_over_prefix": dict(ctx=[2000], nq=[1000], Hq=32, Hkv=4, D=128, Di=64, k=6),
    "g16_d64": dict(ctx=[900, 520], nq=[400, 130], Hq=32, Hkv=2, D=64, Di=128, k=3),
    "g1_d128": dict(ctx=[640], nq=[640], Hq=4, Hkv=4, D=128, Di=128, k=2),
    "g2_k_over_candidates": dict(ctx=[400, 129], nq=[250, 129], Hq=4, Hkv=2, D=64, Di=64, k=8),
    # the largest k and G the library takes: 64 slots per row, 64 parts x 16 heads in the merge
    "k64_g16": dict(ctx=[9000], nq=[300], Hq=32, Hkv=2, D=64, Di=64, k=64),
    # the most KV heads the library takes (64, one query head each) with the largest k
    "hkv64_g1_k64": dict(ctx=[9000], nq=[8], Hq=64, Hkv=64, D=128, Di=64, k=64),
    # many short requests in one chunk: work items from many buckets, rows of many requests
    "many_requests": dict(ctx=[300 + 37 * i for i in range(40)], nq=[1 + (i % 7) * 9 for i in range(40)], Hq=16,
                          Hkv=4, D=128, Di=64, k=3),
    # more (KV head, request, block) buckets than one LDS histogram holds: the remap's global-atomic path
    "remap_many_buckets": dict(ctx=[100000, 90000, 50000], nq=[10, 5, 20], Hq=16, Hkv=8, D=64, Di=64, k=8),
}


def _wl(name, seed=31):
    if CASES[name] is None:
        return mi.tiny_prefill()
    c = dict(CASES[name])
    ctx, nq = c.pop("ctx"), c.pop("nq")
    return mi.small_workload(ctx, nq, seed=seed, **c)


def _run(dev):
    b = batch(dev)
    s = scores(dev, b)
    sel, cnt = topk(dev, b, s)
    po, pl, out, lse = prefill(dev, b, sel, cnt)
    return s, sel, cnt, po, pl, out, lse


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_path_matches_oracle(name):
    announce("prefill", name)
    dev, cpu = setup(_wl(name))
    _check_against_oracle(dev, cpu)


def _check_against_oracle(dev, cpu):
    x = np_inputs(cpu)
    wl = dev.wl
    s, sel, cnt, po, pl, out, lse = [host(t) for t in _run(dev)]

    ref_s = oracle.index_scores(x.q_idx, x.kidx, x.block_table, x.ctx_len, x.q_req, x.q_pos, wl.block)
    assert np.array_equal(np.isneginf(s), np.isneginf(ref_s)), "candidate masks differ"
    fin = np.isfinite(ref_s)
    assert np.abs(s[fin] - ref_s[fin]).max() <= 1e-2

    o_sel, o_cnt = oracle.topk_blocks(s.astype(np.float64), x.q_pos, wl.block, wl.k)
    assert np.array_equal(sel, o_sel) and np.array_equal(cnt, o_cnt), "top-k differs on identical scores"
    r_sel, r_cnt = oracle.topk_blocks(ref_s, x.q_pos, wl.block, wl.k)
    selection_excused(sel, cnt, r_sel, r_cnt, ref_s, wl.k)

    ref_po, ref_pl = oracle.block_partials(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, wl.block, x.scale)
    present = np.arange(wl.k)[None, None, :] < cnt[:, :, None]            # [Nq, Hkv, k]
    assert np.all(np.isneginf(pl[~present])), "empty slots must carry lse = -inf"
    assert_attn_close(po[present], ref_po[present], what="per-block partials")
    assert np.abs(pl[present] - ref_pl[present]).max() <= 1e-3

    ref_o, ref_l = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, wl.block, x.scale)
    assert_attn_close(out, ref_o, what="merged output")
    assert np.abs(lse - ref_l).max() <= 1e-3


TILE_CASES = ["tiny_prefill_2k", "ragged_multi_request", "chunk_over_prefix", "g16_d64", "k64_g16", "many_requests",
              "remap_many_buckets", "g2_k_over_candidates"]


@pytest.mark.parametrize("n_min", [0, 1, 3, 40])
@pytest.mark.parametrize("name", TILE_CASES)
def test_tile_path_matches_oracle(name, n_min):
    """tile_min_rows = n_min: slot_of groups each row's selected slots (only blocks that n_min rows or more
    selected share a slot); every slot holds the oracle's softmax over exactly its group's blocks, the other
    slots of a group lse = -inf; the merged output is the oracle's attention over the selection."""
    announce("prefill tiles", name, f"n_min={n_min}")
    dev, cpu = setup(_wl(name))
    x = np_inputs(cpu)
    wl = dev.wl
    b = batch(dev)
    s = scores(dev, b)
    sel, cnt = topk(dev, b, s)
    slot_of = poison_i32(wl.Nq, wl.Hkv, wl.k)
    po, pl, out, lse = [host(t) for t in prefill(dev, b, sel, cnt, tile_min=n_min, slot_of=slot_of)]
    sel, cnt, slot_of = host(sel), host(cnt), host(slot_of)
    groups = check_slot_of(slot_of, sel, cnt, x.q_req, n_min)
    merged = sum(len(m) > 1 for grp in groups.values() for m in grp.values())
    if n_min in (1, 3) and name in ("tiny_prefill_2k", "chunk_over_prefix", "ragged_multi_request"):
        assert merged > 0, "the tile path merged nothing"
    ref_po, ref_pl = expected_partials(x, sel, cnt, groups)
    present = ~np.isneginf(ref_pl[..., 0])                                 # [Nq, Hkv, k]
    assert np.all(np.isneginf(pl[~present])), "absent and merged-away slots must carry lse = -inf"
    assert_attn_close(po[present], ref_po[present], what="partials")
    assert np.abs(pl[present] - ref_pl[present]).max() <= 1e-3
    ref_o, ref_l = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, wl.block, x.scale)
    assert_attn_close(out, ref_o, what="merged output")
    assert np.abs(lse - ref_l).max() <= 1e-3


def test_tile_path_is_deterministic():
    """Rows are placed in tiles with atomics; results must not depend on that placement."""
    announce("prefill tiles determinism")
    dev, _ = setup(_wl("chunk_over_prefix", seed=8))
    b = batch(dev)
    sel, cnt = topk(dev, b, scores(dev, b))
    a = [host(t) for t in prefill(dev, b, sel, cnt, tile_min=2)]
    for _ in range(3):
        c = [host(t) for t in prefill(dev, b, sel, cnt, tile_min=2)]
        for u, v in zip(a, c):
            fin = ~np.isnan(u)
            assert np.array_equal(u[fin].view(np.uint8), v[fin].view(np.uint8))


def test_prefill_is_deterministic():
    announce("prefill determinism")
    dev, _ = setup(_wl("ragged_multi_request", seed=8))
    a = [host(t) for t in _run(dev)]
    b = [host(t) for t in _run(dev)]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("name", list(CASES))
def test_query_major_matches_oracle(name):
    """The query-major baseline (every (token, KV head) row reads its own k blocks through the
    paged decode kernel) gives the oracle's attention on the same selection, without partials."""
    announce("prefill query-major", name)
    dev, cpu = setup(_wl(name))
    x = np_inputs(cpu)
    wl = dev.wl
    b = batch(dev)
    s = scores(dev, b)
    sel, cnt, pt, rl = topk_page_table(dev, b, s)
    out, lse = decode_attention(dev, pt, rl)
    sel, cnt, out, lse = host(sel), host(cnt), host(out), host(lse)
    o_pt, o_rl = oracle.sparse_page_table(sel, cnt, x.block_table, x.ctx_len, x.q_req, x.q_pos, wl.Hkv, wl.block)
    assert np.array_equal(host(pt), o_pt) and np.array_equal(host(rl), o_rl)
    ref_o, ref_l = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, wl.block, x.scale)
    assert_attn_close(out, ref_o, what="query-major output")
    assert np.abs(lse - ref_l).max() <= 1e-3


WIDE_CASES = {
    # 4 row tiles of 512 x 64 KV heads = 256 workgroups: the scorer takes eight-wave workgroups
    "wide_hkv64_d64": dict(ctx=[2048], nq=[2048], Hq=64, Hkv=64, D=64, Di=64, k=4),
    # three requests in 9 tiles of 512 rows x 32 KV heads, tiles straddling request boundaries, Di = 128
    "wide_ragged_di128": dict(ctx=[3000, 1200, 5000], nq=[1500, 700, 1900], Hq=32, Hkv=32, D=64, Di=128, k=6),
}


def _sample_rows(cu_q, Nq, tile=512, step=37):
    """Rows the oracle checks one by one: every step-th row, both ends of every request and of every
    512-row tile."""
    rows = set(range(0, Nq, step))
    for c in cu_q:
        rows.update(x for x in (c - 1, c) if 0 <= x < Nq)
    for t0 in range(0, Nq, tile):
        rows.update(x for x in (t0 - 1, t0, t0 + 1) if 0 <= x < Nq)
    return np.asarray(sorted(rows))


@pytest.mark.parametrize("name", list(WIDE_CASES))
def test_wide_scorer_workgroups_match_oracle(name):
    """Launches big enough for the eight-wave scorer (one workgroup of 512 rows per CU): block scores
    of sampled rows against the oracle, the fused top-k bit for bit against the oracle's top-k of the
    GPU's own scores, and the two calls' selection identical to the fused one."""
    announce("prefill wide scorer", name)
    c = dict(WIDE_CASES[name])
    ctx, nq = c.pop("ctx"), c.pop("nq")
    dev, cpu = setup(mi.small_workload(ctx, nq, seed=57, **c))
    wl = dev.wl
    x = np_inputs(cpu)
    b = batch(dev)
    s_dev = scores(dev, b)
    s = host(s_dev)
    sel2, cnt2 = topk(dev, b, s_dev)
    msa = lib()
    self_sel, self_cnt = poison_i32(wl.Nq, wl.Hkv, wl.k), poison_i32(wl.Nq, wl.Hkv)
    nws = msa.msa_index_topk_workspace_size(b, wl.Hkv, wl.k)
    assert nws == 0, "k <= 16 runs the fused kernel"
    msa.msa_index_topk(b, dev.q_idx, dev.kidx, wl.k, self_sel, self_cnt, None)
    fsel, fcnt = host(self_sel), host(self_cnt)
    assert np.array_equal(fsel, host(sel2)) and np.array_equal(fcnt, host(cnt2)), "fused and two-call top-k differ"

    rows = _sample_rows(x.cu_q, wl.Nq)
    ref = oracle.index_scores(x.q_idx[rows], x.kidx, x.block_table, x.ctx_len, x.q_req[rows], x.q_pos[rows], wl.block)
    got = s[rows]
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "candidate masks differ"
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() <= 1e-2
    o_sel, o_cnt = oracle.topk_blocks(got.astype(np.float64), x.q_pos[rows], wl.block, wl.k)
    assert np.array_equal(fsel[rows], o_sel) and np.array_equal(fcnt[rows], o_cnt), \
        "fused top-k differs from the oracle's on the GPU's scores"
