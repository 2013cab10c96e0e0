"""msa_index_topk (fused index scoring + top-k) against msa_index_score followed by msa_topk_blocks:
bit-exact selections and counts on every shape -- the fused prefill kernel (k <= 16), and the two-kernel
route it takes for decode shapes and larger k."""
import numpy as np
import pytest
import torch

import msa_inputs as mi
import oracle
from _gpu import announce, batch, host, lib, poison_i32, scores, setup, topk
from _helpers import np_inputs, selection_excused

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_prefill_2k": None,
    "ragged_multi_request_k5": dict(ctx=[700, 300, 1000], nq=[300, 300, 129], Hq=16, Hkv=2, D=128, Di=128, k=5),
    "chunk_over_prefix_k16": dict(ctx=[3000], nq=[1200], Hq=32, Hkv=4, D=128, Di=64, k=16),
    "many_requests_straddling_tiles": dict(ctx=[300, 200, 900, 129, 513], nq=[170, 100, 260, 129, 90], Hq=8, Hkv=2,
                                           D=64, Di=128, k=3),
    "k_over_candidates": dict(ctx=[400, 129], nq=[250, 129], Hq=4, Hkv=2, D=64, Di=64, k=12),
    # exact score ties (bitwise copies of whole blocks) decided by the lower block id inside the fused kernel
    "tied_blocks_k16": dict(ctx=[6000, 2600], nq=[300, 120], Hq=8, Hkv=2, D=64, Di=64, k=16, tie_frac=0.2),
    "k20_two_kernel_route": dict(ctx=[5000], nq=[300], Hq=8, Hkv=2, D=64, Di=64, k=20),
    "decode_two_kernel_route": dict(ctx=[5000, 2049, 777], nq=[1, 3, 1], Hq=16, Hkv=2, D=128, Di=128, k=8),
}


def _wl(name, seed=41):
    if CASES[name] is None:
        return mi.tiny_prefill()
    c = dict(CASES[name])
    ctx, nq = c.pop("ctx"), c.pop("nq")
    return mi.small_workload(ctx, nq, seed=seed, **c)


@pytest.mark.parametrize("name", list(CASES))
def test_index_topk_equals_score_then_topk(name):
    announce("fused index+topk", name)
    msa = lib()
    dev, cpu = setup(_wl(name))
    wl = dev.wl
    b = batch(dev)
    s = scores(dev, b)
    sel_a, cnt_a = topk(dev, b, s)
    sel_b = poison_i32(wl.Nq, wl.Hkv, wl.k)
    cnt_b = poison_i32(wl.Nq, wl.Hkv)
    nws = msa.msa_index_topk_workspace_size(b, wl.Hkv, wl.k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    msa.msa_index_topk(b, dev.q_idx, dev.kidx, wl.k, sel_b, cnt_b, ws)
    sa, ca, sb, cb = host(sel_a), host(cnt_a), host(sel_b), host(cnt_b)
    assert np.array_equal(sa, sb) and np.array_equal(ca, cb)
    # strictly, with no excusal: the oracle's top-k on the GPU's own fp32 scores decides every exact tie
    # at the k-th boundary by the lower block id (tied_blocks_k16 has such ties on many rows)
    o_sel, o_cnt = oracle.topk_blocks(host(s).astype(np.float64), host(dev.q_pos), wl.block, wl.k)
    assert np.array_equal(sa, o_sel) and np.array_equal(ca, o_cnt), "msa_topk_blocks breaks the tie rule"
    assert np.array_equal(sb, o_sel) and np.array_equal(cb, o_cnt), "msa_index_topk breaks the tie rule"
    if name == "tied_blocks_k16":
        assert _boundary_ties(host(s), wl.k) >= 50, "the tie case lost its exact ties at the k-th boundary"
    # and against the oracle's own scores (boundary-excused)
    x = np_inputs(cpu)
    ref_s = oracle.index_scores(x.q_idx, x.kidx, x.block_table, x.ctx_len, x.q_req, x.q_pos, wl.block)
    r_sel, r_cnt = oracle.topk_blocks(ref_s, x.q_pos, wl.block, wl.k)
    selection_excused(sb, cb, r_sel, r_cnt, ref_s, wl.k)


def _boundary_ties(s, k):
    """Rows (t, g) whose k-th and (k+1)-th best scores are exactly equal."""
    n = 0
    for row in s.reshape(-1, s.shape[-1]):
        f = np.sort(row[np.isfinite(row)])[::-1]
        n += int(len(f) > k and f[k - 1] == f[k])
    return n


def test_fused_route_has_no_workspace():
    msa = lib()
    dev, _ = setup(_wl("chunk_over_prefix_k16"))
    assert msa.msa_index_topk_workspace_size(batch(dev), dev.wl.Hkv, 16) == 0
    assert msa.msa_index_topk_workspace_size(batch(dev), dev.wl.Hkv, 17) > 0
