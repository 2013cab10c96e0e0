"""Property tests of the CPU oracle over small random shapes (Hypothesis).

Each property compares an oracle function with something independent of it, over request counts,
context lengths, query counts, head counts, dimensions, k and tie planting drawn at random:
scores against per-token math.fsum loops, the selection against the defining order property,
attention against torch SDPA (float64) with an explicit block mask, the LSE merge of the
per-block partials against one softmax over the union, and the paged decode route (page table
over strided views) against the block-table route.
"""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import msa_inputs as mi
import oracle
from _helpers import np_inputs
from test_oracle_pins import _bruteforce_scores, _sdpa, _topk_by_definition

BS = 16
SETTINGS = settings(max_examples=25, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def workloads(draw, max_ctx=80):
    B = draw(st.integers(1, 3))
    ctx = [draw(st.integers(1, max_ctx)) for _ in range(B)]
    nq = [draw(st.integers(1, min(L, 5))) for L in ctx]
    Hkv = draw(st.integers(1, 3))
    G = draw(st.sampled_from([1, 2, 3]))
    wl = mi.small_workload(ctx, nq, Hq=Hkv * G, Hkv=Hkv, D=draw(st.sampled_from([2, 4, 8])),
                           Di=draw(st.integers(1, 4)), k=draw(st.integers(1, 6)), seed=draw(st.integers(0, 2**31 - 1)),
                           block=BS, tie_frac=draw(st.sampled_from([0.0, 0.25])))
    return np_inputs(mi.make_inputs(wl))


def _scores(x):
    return oracle.index_scores(x.q_idx, x.kidx, x.block_table, x.ctx_len, x.q_req, x.q_pos, BS)


def _select(x):
    s = _scores(x)
    sel, cnt = oracle.topk_blocks(s, x.q_pos, BS, x.wl.k)
    return s, sel, cnt


@SETTINGS
@given(workloads())
def test_scores_match_per_token_loops(x):
    ref = _bruteforce_scores(x)
    got = _scores(x)
    assert np.array_equal(np.isneginf(ref), np.isneginf(got))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=0, atol=1e-11)


@SETTINGS
@given(workloads())
def test_selection_has_the_defining_order_property(x):
    s, sel, cnt = _select(x)
    k = x.wl.k
    for t in range(s.shape[0]):
        n = int(x.q_pos[t]) // BS + 1
        for g in range(s.shape[1]):
            c = int(cnt[t, g])
            chosen = sel[t, g, :c].tolist()
            assert c == min(k, n) and chosen == sorted(chosen) and np.all(sel[t, g, c:] == -1)
            row = s[t, g, :n]
            if n <= 8:
                assert chosen == _topk_by_definition(row, k)
            else:   # every chosen block beats every other candidate under (score desc, id asc)
                rest = [b for b in range(n) if b not in chosen]
                for a in chosen:
                    for b in rest:
                        assert row[a] > row[b] or (row[a] == row[b] and a < b)


@SETTINGS
@given(workloads(max_ctx=60))
def test_attention_matches_block_masked_sdpa(x):
    _, sel, cnt = _select(x)
    out, lse = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                       sel, cnt, BS, x.scale)
    Hkv, G = x.wl.Hkv, x.wl.G
    for t in range(x.q.shape[0]):
        r, p = int(x.q_req[t]), int(x.q_pos[t])
        L = int(x.ctx_len[r])
        tok = np.arange(L)
        K = np.stack([x.kcache[x.block_table[r, s // BS], s % BS] for s in tok]).astype(np.float64)
        V = np.stack([x.vcache[x.block_table[r, s // BS], s % BS] for s in tok]).astype(np.float64)
        for g in range(Hkv):
            chosen = np.isin(tok // BS, sel[t, g, :cnt[t, g]]) & (tok <= p)
            for i in range(G):
                h = g * G + i
                ref = _sdpa(x.q[t, h][None].astype(np.float64), K[:, g], V[:, g], chosen[None], x.scale)[0]
                np.testing.assert_allclose(out[t, h], ref, rtol=0, atol=1e-10)


@SETTINGS
@given(workloads())
def test_merged_block_partials_equal_one_softmax(x):
    _, sel, cnt = _select(x)
    args = (x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos, sel, cnt, BS, x.scale)
    out, lse = oracle.sparse_attention(*args)
    po, pl = oracle.block_partials(*args)
    mo, ml = oracle.lse_merge(po, pl)
    Nq, Hkv, G = x.q.shape[0], x.wl.Hkv, x.wl.G
    np.testing.assert_allclose(mo.reshape(Nq, Hkv * G, -1), out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml.reshape(Nq, Hkv * G), lse, rtol=0, atol=1e-12)


@SETTINGS
@given(workloads())
def test_paged_route_equals_block_table_route(x):
    _, sel, cnt = _select(x)
    out, lse = oracle.sparse_attention(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                       sel, cnt, BS, x.scale)
    Nq, Hkv, G, D = x.q.shape[0], x.wl.Hkv, x.wl.G, x.wl.D
    pt, rl = oracle.sparse_page_table(sel, cnt, x.block_table, x.ctx_len, x.q_req, x.q_pos, Hkv, BS)
    o2, l2 = oracle.paged_decode_attention(x.q.reshape(Nq * Hkv, G, D), x.kcache, x.vcache, pt, rl, D, Hkv * D,
                                           BS, x.scale)
    np.testing.assert_allclose(o2.reshape(out.shape), out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2.reshape(lse.shape), lse, rtol=0, atol=1e-12)
