"""The library keeps no state between calls, so layers enqueued on different streams may run at the
same time: each must reproduce, bit for bit, what it gives when run alone on the default stream."""
import pytest
import torch

import msa_inputs as mi
from _gpu import announce, lib, setup

pytestmark = pytest.mark.gpu


def _layers():
    msa = lib()
    from block_sparse_long_msa_amd.pipeline import MSADecode, MSAPrefill
    made = []
    for wl, prefill in ((mi.small_workload([5000, 2049, 777], [1, 3, 2], Hq=32, Hkv=4, D=128, Di=128, k=8, seed=51),
                         False),
                        (mi.small_workload([3000, 129], [2, 1], Hq=16, Hkv=2, D=64, Di=64, k=5, seed=52), False),
                        (mi.small_workload([1500, 700], [400, 200], Hq=16, Hkv=2, D=128, Di=64, k=6, seed=53), True)):
        dev, _ = setup(wl)
        b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
        cls = MSAPrefill if prefill else MSADecode
        made.append((dev, cls(b, wl.Hkv, wl.G, wl.D, wl.k, dev.kcache.shape[0])))
    return made


def test_layers_on_concurrent_streams_match_their_solo_runs():
    announce("concurrent streams")
    layers = _layers()
    solo = []
    for dev, run in layers:
        out, lse = run(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
        torch.cuda.synchronize()
        solo.append((out.clone(), lse.clone(), run.sel.clone()))
    for rep in range(3):
        for _, run in layers:
            run.out.fill_(float("nan"))
            run.sel.fill_(-7777)
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream() for _ in layers]
        for s, (dev, run) in zip(streams, layers):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                run(dev.q, dev.q_idx, dev.kcache, dev.vcache, dev.kidx, dev.scale)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i, ((out, lse, sel), (_, run)) in enumerate(zip(solo, layers)):
            assert torch.equal(out, run.out) and torch.equal(lse, run.lse) and torch.equal(sel, run.sel), \
                f"repeat {rep}: layer {i} differs when run beside the others"
