"""Benchmark one MSA layer invocation on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload agentic_decode|long_prefill|...]

A step is one pass of the whole MSA hot path over one synthetic batch with every input already
resident in HBM: decode = index scores -> top-k -> sparse page table -> decode attention (+merge);
prefill = index scores -> top-k -> KV-block-major attention -> LSE merge.  Each timed step is
bracketed by HIP events on the stream the kernels run on; a 1 GiB buffer is READ before every
step (outside the events) so that no step finds the previous step's pages in L2 or the MALL (a
write-based flush would leave dirty lines whose write-back competes with the timed kernels).
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import msa_inputs as mi  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
HOST_LINK_PEAK_GBS = 64.0      # PCIe Gen5 x16, one direction, GB/s (K/V read from host memory)
METRIC = "MSA prefill/decode tokens/s; scorer HBM GB/s and attn MFMA % of peak, 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="agentic_decode", choices=sorted(mi.WORKLOADS))
    p.add_argument("--batch", type=int, default=None, help="batch for million_decode (1 or 4)")
    p.add_argument("--no-flush", action="store_true", help="do not read 1 GiB between steps")
    p.add_argument("--cpu-budget-s", type=float, default=12.0, help="oracle time budget for cpu_baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--two-call-topk", action="store_true",
                   help="prefill: always score and select with msa_index_score then msa_topk_blocks (by "
                        "default the fused msa_index_topk runs whenever its launch fills the chip)")
    p.add_argument("--tile-min-rows", type=int, default=None,
                   help="prefill: merge each row's blocks that at least this many rows picked in query tiles "
                        "(0: one partial per selected block; default: the pipeline's)")
    p.add_argument("--prefill-mode", default="kvbm", choices=["kvbm", "query-major"],
                   help="prefill attention: KV-block-major with LSE merge (the method), or the query-major "
                        "baseline it is measured against (each row reads its own blocks)")
    p.add_argument("--decode-select", default="attend", choices=["attend", "page_table", "separate"],
                   help="decode: top-k + page table + attention in one call after the scores (attend), or the "
                        "top-k + page table call then the attention call (page_table), or all three calls")
    p.add_argument("--kv-on-host", action="store_true",
                   help="decode: keep the key-index cache in HBM but move the K/V caches to pinned host memory; "
                        "attention then reads only the selected blocks over the host link")
    p.add_argument("--no-suite", action="store_true",
                   help="time only --workload (by default the other workloads follow, each timed the same way, and "
                        "their per-kernel lines go under 'suite')")
    p.add_argument("--copy-calibration", action="store_true",
                   help="after timing, run one plain 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def make_workload(name, batch):
    if name == "million_decode":
        return mi.million_decode(batch=batch or 1)
    return mi.WORKLOADS[name]()


# --- algorithmic work per launch ----------------------------------------------------------

def recorded_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled against a plain copy), or None when there is none for this
    workload or the kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return rec["traffic_bytes"]


def candidate_tokens(wl):
    """Sum over (query row) of its candidate tokens: tokens 0 .. pos (all valid, pos < L).
    This counts multiply-adds: every query row scores every one of its candidate tokens."""
    total = 0
    for L, nq in zip(wl.ctx_lens, wl.q_counts):
        first = L - nq
        total += sum(p + 1 for p in range(first, L))
    return total


def candidate_tokens_union(wl):
    """Tokens whose key-index rows some query row needs, each counted once per request (the queries of
    one request share their candidate range): the bytes a decode scorer must read."""
    return sum(L for L in wl.ctx_lens)


def selected_tokens(dev, sel, cnt, union: bool = False):
    """Valid tokens over the selected blocks, summed over (query row, KV head); with ``union``, each
    (request, KV head, block) is counted once however many query rows of the request selected it."""
    BS = dev.wl.block
    req = dev.q_req.long()
    lim = torch.minimum(dev.q_pos.long() + 1, dev.ctx_len.long()[req])          # [Nq]
    s = sel.long()
    valid = torch.clamp(lim[:, None, None] - s * BS, min=0, max=BS)
    mask = torch.arange(sel.shape[2], device=sel.device)[None, None, :] < cnt[:, :, None]
    if not union:
        return int((valid * mask).sum().item())
    Nq, Hkv, k = sel.shape
    mb = dev.block_table.shape[1]
    key = (req[:, None, None] * Hkv + torch.arange(Hkv, device=sel.device)[None, :, None]) * mb + s.clamp(min=0)
    best = torch.zeros(dev.wl.B * Hkv * mb, dtype=torch.long, device=sel.device)
    best.scatter_reduce_(0, key[mask], valid[mask], reduce="amax")
    return int(best.sum().item())


# --- cpu_baseline: the CPU oracle, timed on a bounded sample of the same workload ---------------

def cpu_baseline(dev, budget_s: float):
    """Time the CPU oracle (as it stands) on whole query rows of this workload until about
    ``budget_s`` seconds of oracle time are spent, going over the workload again when one pass is
    shorter than that.  Per sampled request the oracle sees only that request's pages, copied to
    host memory outside the timed sections.  The oracle loops over query rows, blocks and heads in
    Python, and each step is a small NumPy product (one 128-token block against one query vector), so
    its time goes to those loops and call overheads, not to BLAS throughput: it runs on one core with
    one BLAS thread, and ``cores`` says so."""
    from threadpoolctl import threadpool_limits

    import oracle
    wl = dev.wl
    BS, Hkv, G, D = wl.block, wl.Hkv, wl.G, wl.D
    host = lambda t: (t.float() if t.is_floating_point() else t).cpu().numpy()
    bt, cu, pos_all = host(dev.block_table), host(dev.cu_q), host(dev.q_pos)
    decode = max(wl.q_counts) <= 16
    spent, tokens, sampled, passes = 0.0, 0, [], 0
    kidx_host = {}                                                          # request -> its K-index pages
    threads = 1
    with threadpool_limits(limits=threads):
        while spent < budget_s:
            passes += 1
            for r in range(wl.B):
                L = wl.ctx_lens[r]
                nb = -(-L // BS)
                if r not in kidx_host:
                    pages = torch.from_numpy(bt[r, :nb].astype(np.int64)).cuda()
                    kidx_host[r] = host(dev.kidx[pages])                        # [nb, BS, Hkv, Di]
                kidx_r = kidx_host[r]
                local_bt = np.arange(nb, dtype=np.int64)[None]
                lo, hi = int(cu[r]), int(cu[r + 1])
                rows = np.arange(lo, hi) if decode else np.linspace(lo, hi - 1, num=min(hi - lo, 4096)).astype(int)
                for c0 in range(0, len(rows), 8):
                    rr = rows[c0:c0 + 8]
                    qi, q, pos = host(dev.q_idx[rr]), host(dev.q[rr]), pos_all[rr]
                    req = np.zeros(len(rr), dtype=np.int64)
                    t0 = time.perf_counter()
                    sc = oracle.index_scores(qi, kidx_r, local_bt, np.asarray([L]), req, pos, BS)
                    sel, cnt = oracle.topk_blocks(sc, pos, BS, wl.k)
                    t1 = time.perf_counter()
                    need = np.unique(sel[sel >= 0])                              # selected blocks' pages only
                    compact = np.zeros((1, nb), dtype=np.int64)
                    compact[0, need] = np.arange(len(need))
                    pg = torch.from_numpy(bt[r, need].astype(np.int64)).cuda()
                    kc, vc = host(dev.kcache[pg]), host(dev.vcache[pg])
                    t2 = time.perf_counter()
                    if decode:
                        pt, rl = oracle.sparse_page_table(sel, cnt, compact, np.asarray([L]), req, pos, Hkv, BS)
                        oracle.paged_decode_attention(q.reshape(len(rr) * Hkv, G, D), kc, vc, pt, rl, D, Hkv * D, BS,
                                                      dev.scale)
                    else:
                        po, pl = oracle.block_partials(q, kc, vc, compact, np.asarray([L]), req, pos, sel, cnt, BS,
                                                       dev.scale)
                        oracle.lse_merge(po, pl)
                    t3 = time.perf_counter()
                    spent += (t1 - t0) + (t3 - t2)
                    tokens += len(rr)
                    sampled.append((r, len(rr)))
                    if spent >= budget_s:
                        break
                if spent >= budget_s:
                    break
    reqs = sorted({r for r, _ in sampled})
    what = (f"{tokens} decode query rows ({len(reqs)} of {wl.B} requests, {passes} pass(es)), all {Hkv} KV heads "
            "and candidate blocks" if decode else
            f"{tokens} prefill query rows (evenly spaced, {passes} pass(es) over up to 4096 of {wl.Nq}), "
            f"all {Hkv} KV heads")
    return {"value": tokens / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}: score, top-k, " + ("page table, paged decode attention" if decode else
                                                     "per-block partials, LSE merge") + f"; {spent:.1f} s",
            "oracle_s": spent}


SUITE = (("tiny_prefill", None), ("long_prefill", None), ("million_decode", 1), ("million_decode", 4),
         ("ragged_decode", None), ("spec_decode", None))


def measure(args, name, batch):
    """Time one workload: W warm-up steps, then K steps bracketed by HIP events, a 1 GiB read before
    every step.  Returns (summary dict, inputs, pipeline)."""
    import block_sparse_long_msa_amd as msa
    from block_sparse_long_msa_amd.pipeline import MSADecode, MSAPrefill, MSAPrefillQueryMajor

    wl = make_workload(name, batch)
    decode = max(wl.q_counts) <= 16
    t0 = time.time()
    dev = mi.make_inputs(wl, "cuda")
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    b = msa.Batch(dev.block_table, dev.ctx_len, dev.cu_q, dev.q_pos, max(wl.q_counts))
    P = dev.kcache.shape[0]
    query_major = not decode and args.prefill_mode == "query-major"
    kv_on_host = decode and args.kv_on_host
    kv_k, kv_v = dev.kcache, dev.vcache
    if kv_on_host:      # pinned host copies; the kernels read them in place over the host link
        kv_k = msa.HostResident(dev.kcache.cpu().pin_memory())
        kv_v = msa.HostResident(dev.vcache.cpu().pin_memory())
    if decode:
        run = MSADecode(b, wl.Hkv, wl.G, wl.D, wl.k, P, select_mode=args.decode_select)
    elif query_major:
        run = MSAPrefillQueryMajor(b, wl.Hkv, wl.G, wl.D, wl.k, P)
    else:
        run = MSAPrefill(b, wl.Hkv, wl.G, wl.D, wl.k, P, fused=False if args.two_call_topk else None,
                         tile_min_rows=args.tile_min_rows)
    flush = None
    if not args.no_flush:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        flush.fill_(1.0)

    def evict():                     # read-only sweep of 1 GiB (one reduction kernel, scalar result)
        flush.sum()

    # stage boundaries for per-kernel event timing
    fused_decode = decode and args.decode_select == "attend"
    stages = (["score", "select_attend"] if fused_decode else
              ["score", "select", "attend"] + ([] if decode or query_major else ["merge"]))

    def step(evs=None):
        for i, stage in enumerate(stages):
            if evs is not None:
                evs[i].record()
            if stage == "score":
                run.score(dev.q_idx, dev.kidx)
            elif stage == "select":
                run.select(kv_k) if (decode or query_major) else run.select()
            elif stage == "attend":
                run.attend(dev.q, kv_k, kv_v, dev.scale)
            elif stage == "select_attend":
                run.select_attend(dev.q, kv_k, kv_v, dev.scale)
            else:
                run.merge()
        if evs is not None:
            evs[-1].record()

    for _ in range(args.warmup):
        if flush is not None:
            evict()
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.time()
    for i in range(args.steps):
        if flush is not None:
            evict()
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.time() - wall0
    per_stage = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(stages))]
                          for i in range(args.steps)])                     # ms
    step_ms = per_stage.sum(axis=1)
    ms_per_step = float(step_ms.mean())
    value = wl.Nq / (ms_per_step / 1e3)

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # roofline of the scorer and of the attention (and merge) kernels
    score_ms = float(per_stage[:, 0].mean())
    attend_ms = float(per_stage[:, stages.index("select_attend" if fused_decode else "attend")].mean())
    cand = candidate_tokens(wl)
    if decode:
        sel_tok = selected_tokens(dev, run.sel, run.cnt, union=True)
        score_bytes = candidate_tokens_union(wl) * wl.Hkv * wl.Di * 2   # every needed k_idx row, once
        roof = {"kernel": "k_score_decode", "bound": "hbm", "achieved": score_bytes / (score_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": recorded_traffic(wl.name),
                "algorithmic_bytes": score_bytes, "avg_ms": score_ms}
        attn_bytes = sel_tok * wl.D * 2 * 2                      # K and V rows of the selected tokens
        if fused_decode:                                         # + the scores the fused top-k reads, once
            attn_bytes += wl.Nq * wl.Hkv * wl.max_blocks * 4
        kname = ("msa_topk_attn_decode (top-k, page table, attention" if fused_decode else "k_attn_decode (attention") + \
            ", split merge)"
        roof_attn = {"kernel": kname, "bound": "host link" if kv_on_host else "hbm",
                     "achieved": attn_bytes / (attend_ms * 1e-3) / 1e9,
                     "peak": HOST_LINK_PEAK_GBS if kv_on_host else HBM_PEAK_GBS, "unit": "GB/s",
                     "algorithmic_bytes": attn_bytes, "avg_ms": attend_ms}
    else:
        sel_tok = selected_tokens(dev, run.sel, run.cnt)
        score_flops = 2.0 * cand * wl.Hkv * wl.Di
        fused_prefill = (not query_major) and run.fused
        roof = {"kernel": "k_score_prefill" + (" with fused top-k" if fused_prefill else ""), "bound": "mfma",
                "achieved": score_flops / (score_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "traffic": None, "algorithmic_flops": score_flops, "avg_ms": score_ms}
        attn_flops = 4.0 * sel_tok * wl.G * wl.D               # QK^T and PV over the selected tokens
        roof_attn = {"kernel": "k_attn_decode (query-major rows)" if query_major else "msa_sparse_attn_prefill",
                     "bound": "mfma", "achieved": attn_flops / (attend_ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "algorithmic_flops": attn_flops, "avg_ms": attend_ms,
                     # K/V bytes the attention mapping moves from memory: query-major reads every
                     # selected block once per (token, KV head) row, KV-block-major once per work item
                     "kv_bytes_moved": sel_tok * wl.D * 2 * 2 if query_major else None}
    details = [roof, roof_attn]
    if not decode and not query_major:
        merge_ms = float(per_stage[:, 3].mean())
        merge_bytes = run.merge_bytes()
        details.append({"kernel": "k_lse_merge<bf16>", "bound": "hbm", "achieved": merge_bytes / (merge_ms * 1e-3) / 1e9,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "algorithmic_bytes": merge_bytes, "avg_ms": merge_ms})
    for r in details:
        r["frac"] = r["achieved"] / r["peak"]
    summary = {
        "workload": wl.name, "phase": "decode" if decode else "prefill", "tokens_per_s": value,
        "ms_per_step": ms_per_step,
        "config": {"workload": wl.name, "phase": "decode" if decode else "prefill", "requests": wl.B,
                   "query_tokens": wl.Nq, "ctx_len": wl.ctx_lens[0] if len(set(wl.ctx_lens)) == 1 else "ragged",
                   "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "Di": wl.Di, "top_k": wl.k, "block": wl.block,
                   "l2_flush_between_steps": flush is not None,
                   "fused_index_topk": bool(not decode and not query_major and run.fused),
                   "prefill_mode": None if decode else args.prefill_mode,
                   "tile_min_rows": None if decode or query_major else run.tile_min_rows,
                   "kv_on_host": bool(kv_on_host),
                   "decode_select": args.decode_select if decode else None},
        "roofline_detail": details,
        "stage_ms": {stage: float(per_stage[:, i].mean()) for i, stage in enumerate(stages)},
        "step_ms_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        "wall_s_timed": wall, "input_gen_s": gen_s,
    }
    return summary, dev, run


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the MSA path would shard "
              "by request or KV head with no exchange; only the one-GPU share is built and timed)",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import block_sparse_long_msa_amd as msa
    msa.load()
    torch.cuda.set_device(0)

    head, dev, run = measure(args, args.workload, args.batch)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dev, budget_s=args.cpu_budget_s)
    del dev, run
    torch.cuda.empty_cache()

    # the other workloads of the same metric, each timed the same way in this run
    suite = []
    if not args.no_suite:
        for name, batch in SUITE:
            if name == args.workload and (batch or 1) == (args.batch or 1):
                continue
            s, dev, run = measure(args, name, batch)
            suite.append({k: s[k] for k in ("workload", "phase", "tokens_per_s", "ms_per_step", "stage_ms",
                                             "roofline_detail", "input_gen_s")})
            print(f"# {s['workload']}: {s['ms_per_step']:.3f} ms per step, "
                  + ", ".join(f"{r['kernel']} {r['frac']:.3f}" for r in s["roofline_detail"]),
                  file=sys.stderr, flush=True)
            del dev, run
            torch.cuda.empty_cache()

    roof = head["roofline_detail"][0]
    line = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": head["config"],
        "roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "roofline_detail": head["roofline_detail"],
        "stage_ms": head["stage_ms"],
        "step_ms_p10_p50_p90": head["step_ms_p10_p50_p90"],
        "cpu_baseline": cpu,
        "wall_s_timed": head["wall_s_timed"], "input_gen_s": head["input_gen_s"],
        "suite": suite,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
