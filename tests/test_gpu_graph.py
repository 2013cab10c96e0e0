"""The decode and prefill pipelines captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every library call launches kernels only (no memsets, no allocation), so a whole MSA layer can be
captured.  Each replay must reproduce the eager step bit for bit; between replays the outputs are
poisoned by eager kernels and the stream is synchronized, so a replay that skipped or mis-ordered a
node could not pass on the eager step's leftovers.
"""
import pytest
import torch

import msa_inputs as mi
from _gpu import announce, lib, setup

pytestmark = pytest.mark.gpu


def _poison(ts):
    for t in ts:
        t.fill_(-7777 if not t.is_floating_point() else float("nan"))


def _check_replays(run, outs, dev):
    args = (dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
    run(*args)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            run(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*args)
    for rep in range(3):
        _poison(outs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outs)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager step"
        run(*args)                      # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["attend", "separate"])
def test_decode_step_replays_from_a_graph(mode):
    announce("graph decode", mode)
    msa = lib()
    from block_sparse_long_msa_amd.pipeline import MSADecode
    wl = mi.small_workload([5000, 2049, 777, 300], [1, 4, 1, 2], Hq=32, Hkv=4, D=128, Di=128, k=8, seed=41)
    dev, _ = setup(wl)
    b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
    run = MSADecode(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0], select_mode=mode)
    _check_replays(run, [run.scores, run.sel, run.cnt, run.page_table, run.row_len, run.out, run.lse], dev)


@pytest.mark.parametrize("fused", [True, False])
def test_prefill_step_replays_from_a_graph(fused):
    announce("graph prefill", "fused" if fused else "two calls")
    msa = lib()
    from block_sparse_long_msa_amd.pipeline import MSAPrefill
    wl = mi.small_workload([900, 2000], [300, 500], Hq=16, Hkv=2, D=128, Di=64, k=6, seed=42)
    dev, _ = setup(wl)
    b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
    run = MSAPrefill(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0], fused=fused)
    # part_o slots of absent parts are never written (their lse is -inf), so they are not compared
    outs = [run.sel, run.cnt, run.part_lse, run.out, run.lse] + ([] if fused else [run.scores])
    _check_replays(run, outs, dev)
