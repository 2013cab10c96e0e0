"""Shared test helpers: tensor -> NumPy conversion for the oracle, tolerance checks."""
from __future__ import annotations

import types

import numpy as np
import torch

import oracle


def np_inputs(inp) -> types.SimpleNamespace:
    """NumPy views of an ``msa_inputs.Inputs`` (bf16 upcast exactly to float32)."""
    f = lambda t: t.detach().to("cpu").float().numpy()
    i = lambda t: t.detach().to("cpu").numpy()
    return types.SimpleNamespace(
        wl=inp.wl, kcache=f(inp.kcache), vcache=f(inp.vcache), kidx=f(inp.kidx), q=f(inp.q),
        q_idx=f(inp.q_idx), block_table=i(inp.block_table), ctx_len=i(inp.ctx_len), cu_q=i(inp.cu_q),
        q_pos=i(inp.q_pos), q_req=i(inp.q_req), scale=inp.scale, hot=inp.hot, ties=inp.ties)


def assert_attn_close(got, ref, atol=2e-2, rtol=1e-2, what="attention"):
    """The attention bar: |got - ref| <= atol + rtol*|ref| elementwise (got upcast from bf16)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref) - (atol + rtol * np.abs(ref))
    bad = np.argwhere(err > 0)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance; first {bad[:5].tolist()}, "
                           f"max abs err {np.abs(got - ref).max():.4g}")


def selection_excused(sel_a, cnt_a, sel_b, cnt_b, scores_ref, k, tol=1e-3):
    """Rows where two selections differ must differ only at the top-k boundary: every block in
    the symmetric difference has a reference score within ``tol`` of the reference k-th score.
    Returns the list of (row, group) pairs that differ (all of them excused) or raises."""
    diff = []
    Nq, Hkv = cnt_a.shape
    for t in range(Nq):
        for g in range(Hkv):
            a = set(int(x) for x in sel_a[t, g, :cnt_a[t, g]])
            b = set(int(x) for x in sel_b[t, g, :cnt_b[t, g]])
            if a == b:
                continue
            s = scores_ref[t, g]
            fin = np.sort(s[np.isfinite(s)])[::-1]
            kth = fin[min(k, len(fin)) - 1]
            for blk in a ^ b:
                assert abs(s[blk] - kth) <= tol, (
                    f"row {t} group {g}: block {blk} differs with score {s[blk]} vs k-th {kth}")
            diff.append((t, g))
    return diff


def block_rows(sel, cnt, q_req):
    """Number of query rows of each (request, KV head) that selected each block: {(r, g, b): rows}."""
    rows = {}
    Nq, Hkv, _ = sel.shape
    for t in range(Nq):
        for g in range(Hkv):
            for j in range(int(cnt[t, g])):
                key = (int(q_req[t]), g, int(sel[t, g, j]))
                rows[key] = rows.get(key, 0) + 1
    return rows


def check_slot_of(slot_of, sel, cnt, q_req, n_min):
    """slot_of as the prefill attention's header states it: -1 past cnt; every selected slot maps to the
    lowest slot of its group, which maps to itself; only blocks that at least n_min rows of the request
    and KV head selected share a slot with others (n_min = 0: every slot is its own).  Returns
    {(t, g): {slot: [member slots]}}."""
    Nq, Hkv, k = sel.shape
    rows = block_rows(sel, cnt, q_req)
    groups = {}
    for t in range(Nq):
        for g in range(Hkv):
            c = int(cnt[t, g])
            assert np.all(slot_of[t, g, c:] == -1), f"row {t} head {g}: slot_of past cnt"
            grp = {}
            for j in range(c):
                s = int(slot_of[t, g, j])
                assert 0 <= s <= j, f"row {t} head {g}: slot {j} maps to {s}"
                grp.setdefault(s, []).append(j)
            for s, members in grp.items():
                assert members[0] == s, f"row {t} head {g}: group {members} not held by its lowest slot"
                if len(members) > 1 or n_min <= 0:
                    assert n_min > 0 or members == [s]
                    for j in members:
                        assert rows[(int(q_req[t]), g, int(sel[t, g, j]))] >= n_min, "ineligible block merged"
            groups[(t, g)] = grp
    return groups


def expected_partials(x, sel, cnt, groups):
    """Per-slot partials the prefill attention must write for the given slot groups: the oracle's softmax
    over the valid keys of every block of a group in the group's slot, lse = -inf in the group's other
    slots (and past cnt)."""
    ref_po, ref_pl = oracle.block_partials(x.q, x.kcache, x.vcache, x.block_table, x.ctx_len, x.q_req, x.q_pos,
                                           sel, cnt, x.wl.block, x.scale)
    G = x.wl.G
    for (t, g), grp in groups.items():
        r, p = int(x.q_req[t]), int(x.q_pos[t])
        for s, members in grp.items():
            if len(members) == 1:
                continue
            blocks = np.asarray([sel[t, g, j] for j in members])
            K, V = oracle.selected_kv(x.kcache, x.vcache, x.block_table[r], blocks, len(blocks), g, p,
                                      int(x.ctx_len[r]), x.wl.block)
            for i in range(G):
                ref_po[t, g, s, i], ref_pl[t, g, s, i] = oracle.attend(x.q[t, g * G + i], K, V, x.scale)
            for j in members[1:]:
                ref_pl[t, g, j, :] = -np.inf
    return ref_po, ref_pl
