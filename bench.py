#!/usr/bin/env python3
"""CSA2 sparse-decode benchmark on one MI355X.

Workload (default): decode batch of 32 sequences at 65,536 tokens (32,768 merged
entries each), 64 query heads, three layers on one cache -- Full (indexer over all
entries, HSI pool of 512 blocks x 8, top-512), Reindex (re-score within the pool),
Reuse (same entries, new query) -- each followed by sparse attention over the 512
selected FP4 entries plus the 128-token bf16 window.  One step also completes the
newest token pair: it merges and writes that pair's entry (the write path) before
the Full layer reads it.  Inputs are seeded synthetic data already resident in HBM;
timed steps rotate over cache replicas so the 256 MB Infinity Cache cannot serve a
step from the previous one.

Prints one JSON line.  `value` = decode queries/s (sequences finishing the
three-layer step per second) with each step replayed as a HIP graph.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-decode queries/s and achieved HBM GB/s (% of peak) at 64K/1M ctx"
HBM_PEAK_GBS = 8000.0           # MI355X published HBM3E bandwidth
BYTES_LAT, BYTES_IDX = 272, 34  # per merged entry (FP4 codes + e8m0 scales)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=8)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seqs", type=int, default=2, help="sequences in the oracle's timed sample")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replay")
    return p.parse_args()


class Replica:
    """One independent copy of the step's inputs (cache + per-layer tensors)."""

    def __init__(self, cache, layers, pair):
        self.cache = cache
        self.layers = layers
        self.pair = pair


def build(case, fk, n_rep: int):
    B = case.B
    dev = "cuda"
    cache = fk.PagedCache.allocate(case.n_pages, case.block_table, device=dev)
    bt_rows = case.block_table.to(dev)
    pair_x, pair_w, pair_k = [], [], []
    for b in range(B):
        x, w, k = case.seq_tokens(b)
        T = x.shape[0]
        sub = fk.PagedCache(cache.lat_codes, cache.lat_scales, cache.idx_codes, cache.idx_scales,
                            bt_rows[b:b + 1].contiguous())
        fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device=dev), x[None].contiguous(),
                    w[None].contiguous(), k[None].contiguous())
        pair_x.append(x[T - 2:].clone())
        pair_w.append(w[T - 2:].clone())
        pair_k.append(k[T // 2 - 1:].clone())
        del x, w, k
    torch.cuda.synchronize()
    pair = dict(x=torch.stack(pair_x).contiguous(), w=torch.stack(pair_w).contiguous(),
                k=torch.stack(pair_k).contiguous(),
                start=torch.tensor([L - 2 for L in case.ctx_len], dtype=torch.int32, device=dev))
    layers = [case.layer(l) for l in range(case.cfg.n_layers)]
    reps = []
    for r in range(n_rep):
        c = cache if r == 0 else cache.clone()
        ls = [{k: (v if r == 0 else v.clone()) for k, v in L.items()} for L in layers]
        pr = {k: (v if r == 0 else v.clone()) for k, v in pair.items()}
        reps.append(Replica(c, ls, pr))
    torch.cuda.synchronize()
    return reps


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on one GPU only (the path has no multi-GPU sharding); "
              f"got --gpus {args.gpus}, WORLD_SIZE={world}", file=sys.stderr)
        return 2
    import fp4_kv_cache_write_amd as fk
    from synth import CONFIGS, make_decode_case

    fk.lib()
    assert torch.cuda.is_available(), "no GPU visible"
    cfg = CONFIGS[1]
    topk, W = cfg.topk, cfg.window
    pool_blocks = cfg.layers[0].pool_blocks
    log(f"building workload {cfg.name} ({args.replicas} replicas)")
    t0 = time.time()
    case = make_decode_case(cfg, device="cuda")
    reps = build(case, fk, args.replicas)
    B, H = case.B, cfg.H
    log(f"built in {time.time() - t0:.1f}s")

    dev = "cuda"
    ctx = torch.tensor(case.ctx_len, dtype=torch.int32, device=dev)
    max_ctx = max(case.ctx_len)
    ws_full = fk.workspace(fk.FN_INDEX_FULL, device=dev, B=B, max_ctx=max_ctx, topk=topk,
                           pool_blocks=pool_blocks)
    tk_full = torch.empty((B, topk), dtype=torch.int32, device=dev)
    tk_re = torch.empty((B, topk), dtype=torch.int32, device=dev)
    pool = torch.empty((B, pool_blocks), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    lses = [torch.empty((B, H), dtype=torch.float32, device=dev) for _ in range(3)]

    def calls(r):
        R = reps[r]
        L = R.layers
        P = R.pair
        return [
            ("write_kv", lambda: fk.write_kv(R.cache, P["start"], P["x"], P["w"], P["k"])),
            ("index_full", lambda: fk.index_full(R.cache, ctx, max_ctx, L[0]["q_idx"], L[0]["w_idx"], topk=topk,
                                                 pool_blocks=pool_blocks, ws=ws_full, topk_idx=tk_full,
                                                 pool=pool)),
            ("sparse_decode", lambda: fk.sparse_decode(R.cache, ctx, L[0]["q"], tk_full, L[0]["swa"],
                                                       out=outs[0], lse=lses[0])),
            ("reindex", lambda: fk.reindex(R.cache, ctx, L[1]["q_idx"], L[1]["w_idx"], pool, topk=topk,
                                           topk_idx=tk_re)),
            ("sparse_decode", lambda: fk.sparse_decode(R.cache, ctx, L[1]["q"], tk_re, L[1]["swa"],
                                                       out=outs[1], lse=lses[1])),
            ("sparse_decode", lambda: fk.sparse_decode(R.cache, ctx, L[2]["q"], tk_re, L[2]["swa"],
                                                       out=outs[2], lse=lses[2])),
        ]

    def run_step(r):
        for _, f in calls(r):
            f()

    # eager warm-up (also sets kernel attributes outside any capture)
    for r in range(len(reps)):
        run_step(r)
    torch.cuda.synchronize()

    # ---- algorithmic bytes per step (formulas in the design doc) ----
    n_vis = case.n_vis
    n_t = [min(topk, v) for v in n_vis]
    n_pool = [min(pool_blocks * cfg.cand_block, v) for v in n_vis]
    n_win = [min(W, L) for L in case.ctx_len]
    by_write = sum(2 * 2 * 1024 + 128 + 4 + 306 for _ in range(B))
    by_full = sum(v * BYTES_IDX + 520 + 4 * topk + 4 * pool_blocks for v in n_vis)
    by_re = sum(p * BYTES_IDX + 520 + 4 * topk + 4 * pool_blocks for p in n_pool)
    by_att = sum(t * BYTES_LAT + w * 1024 + 2 * H * 1024 + 4 * t + 4 * H for t, w in zip(n_t, n_win))
    step_bytes = by_write + by_full + by_re + 3 * by_att
    per_call_bytes = {"write_kv": by_write, "index_full": by_full, "reindex": by_re, "sparse_decode": by_att}

    # ---- graphs: one per replica, each holding one whole step ----
    graphs = []
    use_graph = not args.no_graph
    if use_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            for r in range(len(reps)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    run_step(r)
                graphs.append(g)
            torch.cuda.current_stream().wait_stream(s)
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
        except Exception as e:  # graph capture unavailable: time eager launches
            log(f"graph capture failed ({e!r}); timing eager launches")
            use_graph = False
            graphs = []

    def step(i):
        if use_graph:
            graphs[i % len(graphs)].replay()
        else:
            run_step(i % len(reps))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps ({'graph' if use_graph else 'eager'})")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    ms_step = ev0.elapsed_time(ev1) / args.steps
    ms_step_wall = t_wall * 1e3 / args.steps
    ms = max(ms_step, ms_step_wall)
    qps = B / (ms / 1e3)
    gbs = step_bytes / (ms / 1e3) / 1e9
    log(f"{ms * 1e3:.1f} us/step, {qps:.0f} queries/s, {gbs:.0f} GB/s algorithmic")

    # eager timing for reference
    for i in range(4):
        run_step(i % len(reps))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    n_eager = max(10, args.steps // 4)
    for i in range(n_eager):
        run_step(i % len(reps))
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / n_eager

    # ---- per-call durations: timing events captured between the calls of a step ----
    per_call = {}
    timing_mode = None
    try:
        names = [n for n, _ in calls(0)]
        tg = []
        evs_all = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        for r in range(len(reps)):
            evs = [torch.cuda.Event(enable_timing=True, external=True) for _ in range(len(names) + 1)]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for k, (_, f) in enumerate(calls(r)):
                    evs[k].record()
                    f()
                evs[-1].record()
            tg.append(g)
            evs_all.append(evs)
        torch.cuda.current_stream().wait_stream(s)
        acc = {n: [] for n in set(names)}
        n_rounds = max(4, args.steps // (4 * len(reps)))
        for rnd in range(n_rounds):
            for r, g in enumerate(tg):
                g.replay()
                torch.cuda.synchronize()
                evs = evs_all[r]
                for k, n in enumerate(names):
                    acc[n].append(evs[k].elapsed_time(evs[k + 1]))
        per_call = {n: float(np.mean(v)) for n, v in acc.items()}
        timing_mode = "graph-events"
    except Exception as e:
        log(f"in-graph timing events unavailable ({e!r}); averaging graph replays per call")
        per_call = {}
        try:
            for name in ("write_kv", "index_full", "reindex", "sparse_decode"):
                s = torch.cuda.Stream()
                s.wait_stream(torch.cuda.current_stream())
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for r in range(len(reps)):
                        for n, f in calls(r):
                            if n == name:
                                f()
                                break
                torch.cuda.current_stream().wait_stream(s)
                g.replay()
                torch.cuda.synchronize()
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record()
                for _ in range(8):
                    g.replay()
                a1.record()
                torch.cuda.synchronize()
                per_call[name] = a0.elapsed_time(a1) / (8 * len(reps))
            timing_mode = "graph-replay-average"
        except Exception as e2:
            log(f"per-call timing failed ({e2!r})")
    calls_per_step = {"write_kv": 1, "index_full": 1, "reindex": 1, "sparse_decode": 3}
    roofline = None
    if per_call:
        totals = {n: per_call[n] * calls_per_step[n] for n in per_call}
        dom = max(totals, key=totals.get)
        achieved = per_call_bytes[dom] / (per_call[dom] / 1e3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "avg_launch_us": round(per_call[dom] * 1e3, 2), "timing": timing_mode}
        log("per call (us): " + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per_call.items()))

    # ---- CPU oracle on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, reps[0], topk, W, pool_blocks, args.cpu_seqs)

    line = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "ctx_tokens": max_ctx, "entries_per_seq": max(n_vis),
                   "H": H, "topk": topk, "window": W, "pool_blocks": pool_blocks,
                   "cand_block": cfg.cand_block, "layers": "full,reindex,reuse",
                   "pair_write_per_step": True, "replicas": len(reps),
                   "launch": "hip-graph" if use_graph else "eager"},
        "algorithmic_bytes_per_step": step_bytes,
        "achieved_gbs": round(gbs, 1),
        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "ms_per_step_eager": round(ms_eager, 5),
        "per_call_us": {n: round(v * 1e3, 2) for n, v in per_call.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(case, rep, topk, W, pool_blocks, n_seqs, min_seconds=10.0):
    """Time the NumPy oracle on `n_seqs` sequences of the same inputs (host cores)."""
    from oracle import OracleCache
    from oracle.schedule import run_decode

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max(blas) if blas else 1
    except Exception:
        blas_threads = 1
    seqs = list(range(min(n_seqs, case.B)))
    log(f"cpu baseline: building oracle caches for {len(seqs)} sequence(s) (untimed)")
    caches = {}
    for b in seqs:
        x, w, k = case.seq_tokens(b)
        bt = case.block_table[b:b + 1].numpy()
        oc = OracleCache(case.n_pages, bt)
        T = x.shape[0]
        oc.write(0, 0, bits(x[:T - 2]), bits(w[:T - 2]), bits(k[:T // 2 - 1]))
        caches[b] = (oc, bits(x[T - 2:]), bits(w[T - 2:]), bits(k[T // 2 - 1:]))
    specs = []
    for l, spec in enumerate(case.cfg.layers):
        L = rep.layers[l]
        specs.append(dict(mode=spec.mode, pool_blocks=spec.pool_blocks, q=bits(L["q"]), q_idx=bits(L["q_idx"]),
                          w_idx=bits(L["w_idx"]), swa=bits(L["swa"])))
    log("cpu baseline: timing the oracle")
    t0 = time.perf_counter()
    done = 0
    while True:
        for b in seqs:
            oc, px, pw, pk = caches[b]
            L = case.ctx_len[b]
            oc.write(0, L - 2, px, pw, pk)                   # the step's pair write
            sub = [dict(s, q=s["q"][b:b + 1], q_idx=s["q_idx"][b:b + 1], w_idx=s["w_idx"][b:b + 1],
                        swa=s["swa"][b:b + 1]) for s in specs]
            run_decode(oc, [L], sub, topk=topk, W=W, cand_block=case.cfg.cand_block)
            done += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 3), "unit": "queries/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": f"sequences {seqs} of {case.B} decoded {done // len(seqs)}x each ({done} queries), "
                      f"full 3-layer step incl. pair write, oracle cache pre-built untimed; {dt:.2f}s; "
                      f"numpy float64, BLAS threads={blas_threads}, elementwise single-threaded; "
                      f"host cpus={len(os.sched_getaffinity(0))}"}


if __name__ == "__main__":
    sys.exit(main())
