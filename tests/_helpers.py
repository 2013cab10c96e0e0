"""Shared test helpers: tensor -> NumPy conversion for the oracle, tolerance checks."""
from __future__ import annotations

import types

import numpy as np
import torch


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
