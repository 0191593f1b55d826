#!/usr/bin/env python3
"""CSA2 sparse-decode benchmark on one MI355X.

Headline workload (`value`): decode batch of 32 sequences at 65,536 tokens (32,768
merged entries each), 64 query heads, three layers on one cache -- Full (indexer
over all entries, HSI pool of 512 blocks x 8, top-512), Reindex (re-score within
the pool), Reuse (same entries, new query) -- each followed by sparse attention over
the 512 selected FP4 entries plus the 128-token bf16 window.  One step also
completes the newest token pair: it merges and writes that pair's entry (the write
path) before the Full layer reads it.  Inputs are seeded synthetic data already
resident in HBM; timed steps rotate over cache replicas so the 256 MB Infinity
Cache cannot serve a step from the previous one.  Steps are replayed as HIP graphs.

The same JSON line carries, under "secondary", the single 2K-token query, the 1M-token
decode (8 sequences, Full scan + attention), the chunked prefill (4 x 4,096 queries
against 131,072 prior tokens), the mixed serving batch (128 sequences of 1K-256K
tokens with a 64-token append), the decoder's ratio-1 cache and its 20-layer schedule,
measured the same way.  `--workload` runs one of them alone instead.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
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
MFMA_BF16_PEAK_TFS = 2500.0     # MI355X dense bf16 MFMA
BYTES_LAT, BYTES_IDX = 272, 34  # per merged entry (FP4 codes + e8m0 scales)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=8)
    p.add_argument("--workload", choices=("c0", "c1", "c2", "c3", "c4", "c5"), default="c1",
                   help="c1 = headline decode line (+ secondary c0, c2, c3, c4, c5); others alone")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seqs", type=int, default=2, help="sequences in the headline oracle sample")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="oracle time for the headline line (secondary lines take half)")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replay")
    p.add_argument("--unfused-write", action="store_true",
                   help="run the step's write as its own call instead of inside the first Full layer's scan")
    p.add_argument("--overlap-layers", action="store_true",
                   help="fork each layer's attention onto its own stream (ignores that a layer's queries "
                        "come from the previous layer's output; for reference only)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="first run one 256 MiB device-to-device copy, whose counter readings "
                        "(rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) scale those of the kernels")
    return p.parse_args()


# ----------------------------------------------------------------------------------
# decode workloads
# ----------------------------------------------------------------------------------

class Replica:
    """One independent copy of the step's inputs (cache + per-layer tensors + write)."""

    def __init__(self, cache, layers, write):
        self.cache = cache
        self.layers = layers
        self.write = write


def build_decode(case, fk, n_rep: int):
    """Cache with every sequence's pre-built tokens; the step's write re-submits the
    newest entry's tokens (a pair at ratio 2, one token at ratio 1) when nothing is
    appended, or submits the appended tokens."""
    dev = "cuda"
    cfg = case.cfg
    r = cfg.ratio
    cache = fk.PagedCache.allocate(case.n_pages, case.block_table, device=dev, ratio=r)
    last_x, last_w, last_k = [], [], []
    for b in range(case.B):
        x, w, k = case.seq_tokens(b)
        T = x.shape[0]
        fk.write_kv(cache.rows(b, b + 1), torch.zeros(1, dtype=torch.int32, device=dev), x[None].contiguous(),
                    None if w is None else w[None].contiguous(), k[None].contiguous())
        if cfg.append == 0:
            last_x.append(x[T - r:].clone())
            last_w.append(None if w is None else w[T - r:].clone())
            last_k.append(k[T // r - 1:].clone())
        del x, w, k
    torch.cuda.synchronize()
    if cfg.append == 0:
        write = dict(x=torch.stack(last_x).contiguous(),
                     w=None if r == 1 else torch.stack(last_w).contiguous(),
                     k=torch.stack(last_k).contiguous(),
                     start=torch.tensor([L - r for L in case.ctx_len], dtype=torch.int32, device=dev))
    else:
        xa, wa, ka, start = case.append_tokens()
        write = dict(x=xa.contiguous(), w=None if wa is None else wa.contiguous(), k=ka.contiguous(),
                     start=start.to(dev))
    layers = [case.layer(l) for l in range(cfg.n_layers)]
    reps = []
    for r in range(n_rep):
        c = cache if r == 0 else cache.clone()
        ls = [{k: (v if r == 0 else v.clone()) for k, v in L.items()} for L in layers]
        wr = {k: (v if r == 0 or v is None else v.clone()) for k, v in write.items()}
        reps.append(Replica(c, ls, wr))
    torch.cuda.synchronize()
    return reps


def recorded_traffic(workload: str, call: str):
    """HBM bytes per `call` (FETCH_SIZE + WRITE_SIZE, scaled by the calibration copy) of
    `workload` from the committed counter summaries under profiles/, if they were taken
    on the current sources of that call's kernels (else None)."""
    import glob
    import hashlib
    import re
    pat = re.compile(r"traffic workload=(\S+) call=(\S+) bytes_per_launch=(\d+) sources=(\S+) sha256=([0-9a-f]+)")
    csrc = os.path.join(ROOT, "fp4_kv_cache_write_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_traffic_*.md"))):
        for m in pat.finditer(open(path).read()):
            if m.group(1) != workload or m.group(2) != call:
                continue
            h = hashlib.sha256()
            for f in m.group(4).split(","):
                fp = os.path.join(csrc, f)
                if not os.path.exists(fp):
                    return None
                h.update(open(fp, "rb").read())
            return int(m.group(3)) if h.hexdigest() == m.group(5) else None
    return None


def recorded_mfma_busy(workload: str):
    """MFMA busy % per kernel of `workload` from the committed counter summary under
    profiles/ (SQ_VALU_MFMA_BUSY_CYCLES over active cycles x SIMDs), for kernels whose
    sources still have the recorded hash."""
    import glob
    import hashlib
    import re
    pat = re.compile(r"mfma workload=(\S+) kernel=(\S+) busy_pct=([0-9.]+) sources=(\S+) sha256=([0-9a-f]+)")
    csrc = os.path.join(ROOT, "fp4_kv_cache_write_amd", "csrc")
    out = {}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "pmc_mfma_*.md"))):
        for m in pat.finditer(open(path).read()):
            if m.group(1) != workload:
                continue
            h = hashlib.sha256()
            ok = True
            for f in m.group(4).split(","):
                fp = os.path.join(csrc, f)
                if not os.path.exists(fp):
                    ok = False
                    break
                h.update(open(fp, "rb").read())
            if ok and h.hexdigest() == m.group(5):
                out[m.group(2)] = float(m.group(3))
    return out or None


def decode_bytes(case, fused_write: bool = False):
    """Algorithmic HBM bytes of every call type for one step: each byte a call must
    read or write, counted once.  Full: every visible indexer key (BYTES_IDX each), the
    520 B of indexer query and head weights, the top-K and pool written.  Reindex: the
    pool's keys, the query, the pool read and the top-K written.  Attention: each
    selected latent row (BYTES_LAT), each window row (1 KiB of bf16), the query read and
    the output written (1 KiB per head each), the ids and the per-head log-sum-exp."""
    cfg = case.cfg
    B, H, topk, W = case.B, cfg.H, cfg.topk, cfg.window
    n_vis = case.n_vis
    pool_blocks = max([sp.pool_blocks for sp in cfg.layers] + [0])
    n_t = [min(topk, v) for v in n_vis]
    n_pool = [min(pool_blocks * cfg.cand_block, v) for v in n_vis]
    n_win = [min(W, L) for L in case.ctx_len]
    r = cfg.ratio
    T_w = r if cfg.append == 0 else cfg.append
    per = {   # write reads x (and w at ratio 2) per token and a key per entry, stores 306 B per entry
        "write_kv": B * (T_w * r * 1024 + (T_w // r) * 128 + 4 + (T_w // r) * 306),
        "index_full": sum(v * BYTES_IDX + 520 + 4 * topk + 4 * pool_blocks for v in n_vis),
        "reindex": sum(p * BYTES_IDX + 520 + 4 * pool_blocks + 4 * topk for p in n_pool),
        "sparse_decode": sum(t * BYTES_LAT + w * 1024 + 2 * H * 1024 + 4 * t + 4 * H for t, w in zip(n_t, n_win)),
    }
    count = {"write_kv": 1, "index_full": 0, "reindex": 0, "sparse_decode": 0}
    for sp in cfg.layers:
        count["sparse_decode"] += 1
        if sp.mode == "full":
            count["index_full"] += 1
        elif sp.mode == "reindex":
            count["reindex"] += 1
    if fused_write and cfg.layers[0].mode == "full":
        # the step's write runs inside the first Full layer's scan (csa2_write_index_full)
        per["write_index_full"] = per["write_kv"] + per["index_full"]
        count["write_index_full"] = 1
        count["write_kv"] = 0
        count["index_full"] -= 1
    step = sum(per[n] * count.get(n, 0) for n in per)
    return per, count, step


def bench_decode(fk, cfg_id: int, steps: int, warmup: int, n_rep: int, use_graph: bool, per_call_timing: bool,
                 concurrent: bool = False, fused_write: bool = True):
    from synth import CONFIGS, make_decode_case
    cfg = CONFIGS[cfg_id]
    log(f"building {cfg.name} ({n_rep} replicas)")
    t0 = time.time()
    case = make_decode_case(cfg, device="cuda")
    reps = build_decode(case, fk, n_rep)
    log(f"built in {time.time() - t0:.1f}s")
    dev = "cuda"
    B, H, topk = case.B, cfg.H, cfg.topk
    ctx = torch.tensor(case.ctx_len, dtype=torch.int32, device=dev)
    max_ctx = max(case.ctx_len)
    pool_blocks = max([sp.pool_blocks for sp in cfg.layers] + [0])
    ws_full = fk.workspace(fk.FN_INDEX_FULL, device=dev, B=B, max_ctx=max_ctx, topk=topk, pool_blocks=pool_blocks,
                           ratio=cfg.ratio)
    ws_re = fk.workspace(fk.FN_REINDEX, device=dev, B=B, topk=topk, pool_blocks=max(pool_blocks, 1),
                         ratio=cfg.ratio)
    ws_att = fk.workspace(fk.FN_SPARSE_DECODE, device=dev, B=B, H=H, topk=topk)
    tk_buf = [torch.empty((B, topk), dtype=torch.int32, device=dev) for _ in range(2)]
    pool = torch.empty((B, max(pool_blocks, 1)), dtype=torch.int32, device=dev)
    outs = [torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev) for _ in cfg.layers]
    lses = [torch.empty((B, H), dtype=torch.float32, device=dev) for _ in cfg.layers]

    def calls(r):
        R = reps[r]
        Wr = R.write
        fuse = fused_write and cfg.layers[0].mode == "full"
        out = [] if fuse else [("write_kv", lambda: fk.write_kv(R.cache, Wr["start"], Wr["x"], Wr["w"], Wr["k"]))]
        cur = None
        nxt = 0
        for l, sp in enumerate(cfg.layers):
            L = R.layers[l]
            if sp.mode == "full" and l == 0 and fuse:
                tk = tk_buf[nxt]
                nxt ^= 1
                pb = sp.pool_blocks
                out.append(("write_index_full", lambda L=L, tk=tk, pb=pb: fk.write_index_full(
                    R.cache, Wr["start"], Wr["x"], Wr["w"], Wr["k"], ctx, max_ctx, L["q_idx"], L["w_idx"],
                    topk=topk, pool_blocks=pb, cand_block=cfg.cand_block, ws=ws_full, topk_idx=tk,
                    pool=pool if pb > 0 else None)))
                cur = tk
            elif sp.mode == "full":
                tk = tk_buf[nxt]
                nxt ^= 1
                pb = sp.pool_blocks
                out.append(("index_full", lambda L=L, tk=tk, pb=pb: fk.index_full(
                    R.cache, ctx, max_ctx, L["q_idx"], L["w_idx"], topk=topk, pool_blocks=pb,
                    cand_block=cfg.cand_block, ws=ws_full, topk_idx=tk, pool=pool if pb > 0 else None)))
                cur = tk
            elif sp.mode == "reindex":
                tk = tk_buf[nxt]
                nxt ^= 1
                out.append(("reindex", lambda L=L, tk=tk: fk.reindex(R.cache, ctx, L["q_idx"], L["w_idx"], pool,
                                                                     topk=topk, cand_block=cfg.cand_block,
                                                                     topk_idx=tk, ws=ws_re)))
                cur = tk
            out.append(("sparse_decode", lambda L=L, tk=cur, l=l: fk.sparse_decode(
                R.cache, ctx, L["q"], tk, L["swa"], out=outs[l], lse=lses[l], ws=ws_att)))
        return out

    # Default: the step's calls run in layer order on one stream, as a model must run
    # them (layer l+1's indexer and attention queries come from layer l's output).
    # With concurrent=True the selector chain (write, Full, Reindex) stays on the
    # launching stream and each layer's attention is forked onto a stream of its own;
    # that overlaps layers a model cannot overlap and is kept only for reference.
    side = [torch.cuda.Stream() for _ in cfg.layers] if concurrent else []

    def run_step(r):
        if not concurrent:
            for _, f in calls(r):
                f()
            return
        main = torch.cuda.current_stream()
        layer = 0
        for name, f in calls(r):
            if name == "sparse_decode":
                s = side[layer]
                s.wait_stream(main)
                with torch.cuda.stream(s):
                    f()
                layer += 1
            else:
                f()
        for s in side:
            main.wait_stream(s)

    for r in range(len(reps)):          # eager warm-up (sets kernel attributes outside capture)
        run_step(r)
    torch.cuda.synchronize()

    per_bytes, count, step_bytes = decode_bytes(case, fused_write)
    graphs = []
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
        except Exception as e:
            log(f"graph capture failed ({e!r}); timing eager launches")
            use_graph, graphs = False, []

    def step(i):
        if use_graph:
            graphs[i % len(graphs)].replay()
        else:
            run_step(i % len(reps))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record()
    for i in range(steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    ms = max(ev0.elapsed_time(ev1) / steps, t_wall * 1e3 / steps)
    qps = B / (ms / 1e3)
    gbs = step_bytes / (ms / 1e3) / 1e9
    log(f"{cfg.name}: {ms * 1e3:.1f} us/step, {qps:.0f} queries/s, {gbs:.0f} GB/s algorithmic")

    per_call = {}
    if per_call_timing:
        # each call type alone: a graph holding that call once per replica, replayed 8 times
        # (launched and timed on the current stream)
        for name in [n for n in ("write_kv", "write_index_full", "index_full", "reindex", "sparse_decode")
                     if count.get(n, 0) > 0]:
            try:
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
            except Exception as e:
                log(f"per-call timing of {name} failed ({e!r})")
        log("per call (us): " + ", ".join(f"{n}={v * 1e3:.1f}" for n, v in per_call.items()))
    roofline = None
    if per_call:
        totals = {n: per_call[n] * count[n] for n in per_call}
        dom = max(totals, key=totals.get)
        achieved = per_bytes[dom] / (per_call[dom] / 1e3) / 1e9
        traffic = recorded_traffic(cfg.name, dom)
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "bytes_per_launch": per_bytes[dom], "avg_launch_us": round(per_call[dom] * 1e3, 2),
                    "timing": "graph replay of that call, averaged per launch"}
    return dict(case=case, reps=reps, ms=ms, qps=qps, gbs=gbs, step_bytes=step_bytes, per_call=per_call,
                roofline=roofline, use_graph=use_graph, count=count, per_bytes=per_bytes)


def bench_schedule(fk, cfg_id: int, schedule, steps: int, warmup: int, n_rep: int = 4, cpu_seqs=(),
                   cpu_seconds=5.0):
    """One decode step of a whole layer schedule through the native runner
    (csa2_schedule_*: the step's write plus every layer captured as one HIP graph),
    replayed over n_rep cache replicas."""
    import dataclasses
    from synth import CONFIGS, make_decode_case
    cfg = dataclasses.replace(CONFIGS[cfg_id], layers=tuple(schedule),
                              name=CONFIGS[cfg_id].name + f"_schedule{len(schedule)}")
    log(f"building {cfg.name} ({n_rep} replicas, native schedule runner)")
    case = make_decode_case(cfg, device="cuda")
    reps = build_decode(case, fk, n_rep)
    dev = "cuda"
    B, H = case.B, cfg.H
    ctx = torch.tensor(case.ctx_len, dtype=torch.int32, device=dev)
    outs = [torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev) for _ in cfg.layers]
    scheds = []
    for R in reps:
        layers = [dict(mode=sp.mode, pool_blocks=sp.pool_blocks, q=R.layers[l]["q"], q_idx=R.layers[l]["q_idx"],
                       w_idx=R.layers[l]["w_idx"], swa=R.layers[l]["swa"], out=outs[l])
                  for l, sp in enumerate(cfg.layers)]
        scheds.append(fk.Schedule(R.cache, ctx, max(case.ctx_len), layers, W=cfg.window, topk=cfg.topk,
                                  cand_block=cfg.cand_block, write=R.write))
    for i in range(warmup):
        scheds[i % n_rep].launch()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(steps):
        scheds[i % n_rep].launch()
    ev1.record()
    torch.cuda.synchronize()
    ms = max(ev0.elapsed_time(ev1) / steps, (time.perf_counter() - t0) * 1e3 / steps)
    _, count, step_bytes = decode_bytes(case)
    for sc in scheds:
        sc.close()
    log(f"{cfg.name}: {ms * 1e3:.1f} us/step ({len(cfg.layers)} layers), {B / (ms / 1e3):.0f} queries/s")
    cpu = (cpu_baseline_decode(case, reps[0], cpu_seqs, cpu_seconds, f"{len(cpu_seqs)} of {B} sequences")
           if cpu_seqs else None)
    return {"workload": cfg.name, "value": round(B / (ms / 1e3), 1), "unit": "queries/s",
            "ms_per_step": round(ms, 5), "layers": len(cfg.layers), "us_per_layer": round(ms * 1e3 / len(cfg.layers), 2),
            "achieved_gbs": round(step_bytes / (ms / 1e3) / 1e9, 1), "algorithmic_bytes_per_step": step_bytes,
            "launch": "native schedule runner: write + all layers as one HIP graph", "cpu_baseline": cpu}


# ----------------------------------------------------------------------------------
# chunked prefill
# ----------------------------------------------------------------------------------

def bench_prefill(fk, steps: int, warmup: int, cpu_seqs=()):
    from synth import CONFIGS, make_prefill_case
    cfg = CONFIGS[3]
    dev = "cuda"
    log(f"building {cfg.name}")
    case = make_prefill_case(cfg, dev)
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device=dev)
    bt = case.block_table.to(dev)
    for b in range(case.B):
        x, w, k = case.prior_tokens(b)
        sub = fk.PagedCache(gc.lat_codes, gc.lat_scales, gc.idx_codes, gc.idx_scales, bt[b:b + 1].contiguous())
        fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device=dev), x[None].contiguous(), w[None].contiguous(),
                    k[None].contiguous())
        del x, w, k
    ch = case.chunk()
    prior = torch.full((case.B,), cfg.prior, dtype=torch.int32, device=dev)
    start = ch["start_tok"].to(dev)
    max_ctx = cfg.prior + cfg.C
    out = torch.empty((case.B, cfg.C, cfg.H, 512), dtype=torch.bfloat16, device=dev)
    tk = torch.empty((case.B, cfg.C, cfg.topk), dtype=torch.int32, device=dev)
    ws = fk.workspace(fk.FN_PREFILL_CHUNK, device=dev, B=case.B, H=cfg.H, max_ctx=max_ctx, topk=cfg.topk, C=cfg.C)

    def write():
        fk.write_kv(gc, start, ch["x"], ch["w"], ch["k_idx"])

    def attend():
        fk.prefill_chunk(gc, prior, max_ctx, ch["q"], ch["q_idx"], ch["w_idx"], ch["local"], topk=cfg.topk,
                         out=out, topk_idx=tk, ws=ws)

    for _ in range(warmup):
        write()
        attend()
    torch.cuda.synchronize()
    # Steps queued back to back (one synchronisation at the end), so no host latency
    # falls between the events; the indexer + attention part is timed here, the write
    # below.
    evs = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        write()
        e[1].record()
        attend()
        e[2].record()
        evs.append(e)
    torch.cuda.synchronize()
    ms_a = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    e = evs[0]

    # The write alone, per launch: one HIP graph of launches over 10 copies of the
    # chunk's inputs (10 x 33.6 MB, more than the 256 MB Infinity Cache), so that every
    # launch reads its inputs from HBM and no host call sits between launches.
    n_copy = 10
    copies = [(ch["x"].clone(), ch["w"].clone(), ch["k_idx"].clone()) for _ in range(n_copy)]
    for xc, wc, kc in copies:
        fk.write_kv(gc, start, xc, wc, kc)
    torch.cuda.synchronize()
    gs = torch.cuda.Stream()
    gs.wait_stream(torch.cuda.current_stream())
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw, stream=gs):
        for xc, wc, kc in copies:
            fk.write_kv(gc, start, xc, wc, kc)
    torch.cuda.current_stream().wait_stream(gs)
    gw.replay()
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(steps):
        gw.replay()
    e[1].record()
    torch.cuda.synchronize()
    ms_w = e[0].elapsed_time(e[1]) / (steps * n_copy)
    del gw, copies
    ms = ms_w + ms_a

    # The same chunk written with its indexer keys projected from the entries by a
    # seeded bf16 [64][512] weight matrix (csa2_write_kv_proj), timed on its own.
    gen = torch.Generator().manual_seed(cfg.seed + 77)
    w_proj = (torch.randn((64, 512), generator=gen) / 512 ** 0.5).to(torch.bfloat16).to(dev)

    def write_proj():
        fk.write_kv_proj(gc, start, ch["x"], ch["w"], w_proj)

    for _ in range(3):
        write_proj()
    torch.cuda.synchronize()
    e[0].record()
    for _ in range(steps):
        write_proj()
    e[1].record()
    torch.cuda.synchronize()
    ms_wp = e[0].elapsed_time(e[1]) / steps
    n_ent = case.B * cfg.C // 2
    wp_bytes = n_ent * (4 * 1024 + 306) + 64 * 512 * 2       # x, w of two tokens in; entry out; weights once
    write_proj_line = {"us": round(ms_wp * 1e3, 2), "entries": n_ent,
                       "achieved_gbs": round(wp_bytes / (ms_wp / 1e3) / 1e9, 1),
                       "fp64_gflops": round(n_ent * 64 * 512 * 2 / (ms_wp / 1e3) / 1e9, 1),
                       "write_with_supplied_keys_us": round(ms_w * 1e3, 2)}
    log(f"{cfg.name}: write with projected keys {ms_wp * 1e3:.1f} us for {n_ent} entries "
        f"(supplied keys: {ms_w * 1e3:.1f} us per launch, graph replay, inputs from HBM)")
    nv = (cfg.prior + np.arange(cfg.C) + 1) // 2
    n_win = np.minimum(cfg.window, cfg.prior + np.arange(cfg.C) + 1)
    fl_idx = case.B * float(np.sum(nv)) * 4 * 64 * 2
    fl_att = case.B * float(np.sum(cfg.H * (np.minimum(nv, cfg.topk) + n_win) * 512 * 2 * 2))
    tfs = (fl_idx + fl_att) / (ms_a / 1e3) / 1e12
    toks = case.B * cfg.C / (ms / 1e3)
    log(f"{cfg.name}: write {ms_w * 1e3:.0f} us + prefill {ms_a * 1e3:.0f} us; {toks:.0f} tokens/s, "
        f"{tfs:.1f} TFLOP/s")
    cpu = None
    if cpu_seqs:
        cpu = cpu_baseline_prefill(case, ch, cpu_seqs, 64, f"{len(cpu_seqs)} of {case.B} chunks")
        log(f"{cfg.name}: oracle {cpu['value']} tokens/s (extrapolated)")
    return {"workload": cfg.name, "metric": "prefill query tokens/s", "value": round(toks, 1),
            "unit": "tokens/s", "ms_per_step": round(ms, 4), "ms_write": round(ms_w, 4),
            "write_gbs": round(n_ent * (4 * 1024 + 128 + 306) / (ms_w / 1e3) / 1e9, 1),
            "ms_index_attention": round(ms_a, 4), "flop_indexer": fl_idx, "flop_attention": fl_att,
            "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                         "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                         "mfma_busy_pct_counters": recorded_mfma_busy(cfg.name)},
            "write_proj": write_proj_line, "dtype": "bf16", "steps": steps, "warmup": warmup,
            "cpu_baseline": cpu}


def bench_hisa(fk, steps: int, warmup: int, n_rep: int = 4, cfg_id: int = 1, cpu_seqs=(), cpu_seconds=5.0):
    """HISA selection at a decode workload's size (blocks of 8 entries): per
    step, the newest block's summary is refreshed (csa2_block_keys) and the 512 best
    block summaries are expanded and re-scored to the top-512 (csa2_index_full on the
    block cache, then csa2_reindex); timed beside the Full layer's selection with its
    HSI pool of the same size, as HIP-graph replays over cache replicas."""
    from synth import CONFIGS, make_decode_case
    cfg = CONFIGS[cfg_id]
    dev = "cuda"
    case = make_decode_case(cfg, device=dev)
    reps = build_decode(case, fk, n_rep)
    B, topk, cb, keep = case.B, cfg.topk, cfg.cand_block, 512
    ctx = torch.tensor(case.ctx_len, dtype=torch.int32, device=dev)
    max_ctx = max(case.ctx_len)
    nb_max = -(-(max_ctx // 2) // cb)
    P = -(-nb_max // 64)
    bt = torch.arange(B * P, dtype=torch.int32, device=dev).reshape(B, P)
    blocks = [fk.PagedCache.allocate(B * P, bt, device=dev, ratio=1) for _ in reps]
    nbs = [fk.block_keys(R.cache, bk, ctx, max_ctx, cand_block=cb) for R, bk in zip(reps, blocks)]
    newest = torch.tensor([(L // 2 - 1) // cb for L in case.ctx_len], dtype=torch.int32, device=dev)
    ws_b = fk.workspace(fk.FN_INDEX_FULL, device=dev, B=B, max_ctx=nb_max, topk=keep, pool_blocks=0, ratio=1)
    ws_r = fk.workspace(fk.FN_REINDEX, device=dev, B=B, topk=topk, pool_blocks=keep, ratio=2)
    # the Full layer's own HSI pool ranks up to 32768 blocks; past that it selects without one
    pb = keep if -(-(max_ctx // 2) // cb) <= 32768 else 0
    ws_f = fk.workspace(fk.FN_INDEX_FULL, device=dev, B=B, max_ctx=max_ctx, topk=topk, pool_blocks=pb, ratio=2)
    tk = torch.empty((B, topk), dtype=torch.int32, device=dev)
    pool = torch.empty((B, keep), dtype=torch.int32, device=dev)

    def hisa(r):
        L = reps[r].layers[0]
        fk.block_keys(reps[r].cache, blocks[r], ctx, max_ctx, cand_block=cb, blk_first=newest, n_span=1,
                      n_blocks=nbs[r])
        fk.index_hisa(reps[r].cache, blocks[r], nbs[r], nb_max, ctx, L["q_idx"], L["w_idx"], keep_blocks=keep,
                      topk=topk, cand_block=cb, ws_blocks=ws_b, ws_reindex=ws_r)

    def full(r):
        L = reps[r].layers[0]
        fk.index_full(reps[r].cache, ctx, max_ctx, L["q_idx"], L["w_idx"], topk=topk, pool_blocks=pb,
                      cand_block=cb, ws=ws_f, topk_idx=tk, pool=pool if pb else None)

    out = {}
    for name, f in (("hisa", hisa), ("full", full)):
        for r in range(n_rep):
            f(r)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for r in range(n_rep):
                f(r)
        torch.cuda.current_stream().wait_stream(s)
        for _ in range(max(1, warmup)):
            g.replay()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(steps):
            g.replay()
        a1.record()
        torch.cuda.synchronize()
        out[name] = a0.elapsed_time(a1) / (steps * n_rep) * 1e3
    n_vis = case.n_vis
    hisa_bytes = sum((-(-v // cb)) * BYTES_IDX + keep * cb * BYTES_IDX + 2 * 520 + 4 * topk for v in n_vis)
    log(f"{cfg.name} HISA selection {out['hisa']:.1f} us/step vs Full{' + HSI pool' if pb else ''} {out['full']:.1f} us")
    cpu = cpu_baseline_hisa(case, cpu_seqs, reps[0].layers[0], keep, cpu_seconds) if cpu_seqs else None
    return {"workload": f"{cfg.name.split('_h64')[0]}_hisa_blocks{cb}_keep{keep}", "us_per_step": round(out["hisa"], 2),
            "full_selection_us": round(out["full"], 2), "full_selection_has_pool": bool(pb),
            "value": round(B / (out["hisa"] / 1e6), 1),
            "unit": "selections/s", "algorithmic_bytes_per_step": hisa_bytes,
            "achieved_gbs": round(hisa_bytes / (out["hisa"] / 1e6) / 1e9, 1),
            "launch": "hip-graph; block_keys (newest block) + index_full over block summaries + reindex",
            "cpu_baseline": cpu}


# ----------------------------------------------------------------------------------

def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU only (the path has no multi-GPU sharding); "
              f"got --gpus {args.gpus}, WORLD_SIZE={world}", file=sys.stderr)
        return 2
    import fp4_kv_cache_write_amd as fk
    fk.lib()
    assert torch.cuda.is_available(), "no GPU visible"
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")    # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 268435456 bytes read, 268435456 bytes written")
        del src, dst

    if args.workload == "c3":
        r = bench_prefill(fk, max(2, args.steps // 40), max(1, args.warmup // 10),
                          cpu_seqs=() if args.no_cpu_baseline else (0, 3))
        print(json.dumps(dict(r, n_gpus=1, higher_is_better=True, data="synthetic", vs_baseline=None,
                              config={"workload": r["workload"]})), flush=True)
        return 0

    cfg_id = {"c0": 0, "c1": 1, "c2": 2, "c4": 4, "c5": 5}[args.workload]
    fused = not args.unfused_write
    d = bench_decode(fk, cfg_id, args.steps, args.warmup, args.replicas, not args.no_graph, True, args.overlap_layers,
                     fused)
    case = d["case"]
    cfg = case.cfg
    secondary = {}
    want_cpu = not args.no_cpu_baseline
    sec_s = args.cpu_seconds / 2
    if args.workload == "c1" and not args.no_secondary:
        def decode_line(cid, n_rep, cpu_seqs):
            r = bench_decode(fk, cid, max(20, args.steps // 4), max(5, args.warmup // 4), n_rep, not args.no_graph,
                             True, args.overlap_layers, fused)
            c = r["case"]
            out = {"workload": c.cfg.name, "value": round(r["qps"], 1), "unit": "queries/s",
                   "ms_per_step": round(r["ms"], 5), "achieved_gbs": round(r["gbs"], 1),
                   "frac_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": r["step_bytes"],
                   "per_call_us": {n: round(v * 1e3, 2) for n, v in r["per_call"].items()}, "roofline": r["roofline"],
                   "cpu_baseline": None}
            if want_cpu:
                seqs = cpu_seqs(c)
                out["cpu_baseline"] = cpu_baseline_decode(c, r["reps"][0], seqs, sec_s,
                                                          f"{len(seqs)} of {c.B} sequences")
            del r
            torch.cuda.empty_cache()
            return out

        def seeded(n, seed):
            return lambda c: tuple(sorted(np.random.default_rng(seed).choice(c.B, size=n, replace=False).tolist()))

        # a single 2K-token query: launch-latency bound, reported for completeness
        secondary["c0_b1_ctx2k"] = decode_line(0, 8, lambda c: (0,))
        secondary["c2_b8_ctx1m"] = decode_line(2, 4, seeded(1, 2002))
        secondary["c3_prefill"] = bench_prefill(fk, 5, 2, cpu_seqs=(0, 3) if want_cpu else ())
        torch.cuda.empty_cache()
        # mixed serving batch: 128 sequences of log-uniform length, 64-token append per step;
        # the oracle's sample is 8 sequences drawn uniformly, so its queries/s is unbiased
        secondary["c4_b128_mixed"] = decode_line(4, 2, seeded(8, 2004))
        # the decoder's ratio-1 cache with the 2048-block HSI pool
        secondary["c5_decoder_ratio1"] = decode_line(5, 4, seeded(2, 2005))
        # HISA's block-mean pool as the selection, beside the Full layer's
        secondary["c1_hisa"] = bench_hisa(fk, max(20, args.steps // 4), max(5, args.warmup // 4),
                                          cpu_seqs=(0, 31) if want_cpu else (), cpu_seconds=sec_s)
        torch.cuda.empty_cache()
        secondary["c2_hisa"] = bench_hisa(fk, max(20, args.steps // 4), max(5, args.warmup // 4), n_rep=2, cfg_id=2,
                                          cpu_seqs=(5,) if want_cpu else (), cpu_seconds=sec_s)
        torch.cuda.empty_cache()
        # the pages' whole decoder schedule (20 layers) at that size, through the native runner
        from synth.configs import DECODER_SCHEDULE
        secondary["c5_decoder_schedule20"] = bench_schedule(fk, 5, DECODER_SCHEDULE, max(10, args.steps // 10),
                                                            max(3, args.warmup // 4),
                                                            cpu_seqs=(7,) if want_cpu else (), cpu_seconds=sec_s)
        torch.cuda.empty_cache()

    cpu = None
    if want_cpu and args.workload != "c3":
        n = max(1, min(args.cpu_seqs, case.B))
        seqs = tuple(sorted({int(round(i * (case.B - 1) / max(n - 1, 1))) for i in range(n)}))
        cpu = cpu_baseline_decode(case, d["reps"][0], seqs, args.cpu_seconds, f"{len(seqs)} of {case.B} sequences")

    line = {
        "metric": METRIC,
        "value": round(d["qps"], 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": case.B, "ctx_tokens": max(case.ctx_len),
                   "entries_per_seq": max(case.n_vis), "H": cfg.H, "topk": cfg.topk, "window": cfg.window,
                   "pool_blocks": max([sp.pool_blocks for sp in cfg.layers] + [0]), "cand_block": cfg.cand_block,
                   "layers": ",".join(sp.mode for sp in cfg.layers), "write_per_step": True,
                   "write": ("inside the first Full layer's scan (csa2_write_index_full)"
                             if fused and cfg.layers[0].mode == "full" else "its own call (csa2_write_kv)"),
                   "replicas": len(d["reps"]), "launch": ("hip-graph" if d["use_graph"] else "eager") +
                   ("; each layer's attention on its own forked stream (layers overlapped)" if args.overlap_layers
                    else "; layers in order on one stream")},
        "algorithmic_bytes_per_step": d["step_bytes"],
        "achieved_gbs": round(d["gbs"], 1),
        "frac_hbm_peak": round(d["gbs"] / HBM_PEAK_GBS, 4),
        "per_call_us": {n: round(v * 1e3, 2) for n, v in d["per_call"].items()},
        "roofline": d["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary or None,
    }
    print(json.dumps(line), flush=True)
    return 0


# ----------------------------------------------------------------------------------
# the CPU oracle as a reported baseline (bounded samples of the same workloads)
# ----------------------------------------------------------------------------------

def _host_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _host_threads():
    """(cpus this process may run on, BLAS threads numpy uses)."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        blas_threads = max(blas) if blas else 1
    except Exception:
        blas_threads = 1
    return len(os.sched_getaffinity(0)), blas_threads


def _seq_table(case, b, n_entries=None):
    """Sequence b's own pages renumbered 0..P-1 in the same relative order, so that an
    oracle cache for one sequence holds only that sequence's pages."""
    row = case.block_table[b].numpy()
    if n_entries is None:
        n_entries = case.ctx_len[b] // case.cfg.ratio
    P = -(-n_entries // 64)
    row = row[:max(P, 1)]
    return np.argsort(np.argsort(row))[None, :], max(P, 1)


def _oracle_decode_caches(case, rep, seqs, specs):
    """Per sampled sequence, an oracle cache ready for the timed step (untimed set-up):
    every indexer key before the step's write, then, from a dry run of the oracle's own
    layers, the latent rows those layers read.  The step's write is re-done when timed."""
    from oracle import OracleCache
    from oracle.schedule import run_decode
    cfg = case.cfg
    r = cfg.ratio
    Wr = rep.write
    out = {}
    for b in seqs:
        bt, P = _seq_table(case, b)
        oc = OracleCache(P, bt, ratio=r)
        x, w, k = case.seq_tokens(b)
        start = int(Wr["start"][b])
        n_pre = start // r
        oc.write(0, 0, None, None, _host_bits(k[:n_pre]), latent=False)
        wx = _host_bits(Wr["x"][b])
        ww = None if Wr["w"] is None else _host_bits(Wr["w"][b])
        wk = _host_bits(Wr["k"][b])
        oc.write(0, start, wx, ww, wk)
        sub = [dict(s, q=s["q"][b:b + 1], q_idx=s["q_idx"][b:b + 1], w_idx=s["w_idx"][b:b + 1],
                    swa=s["swa"][b:b + 1]) for s in specs]
        dry = run_decode(oc, [case.ctx_len[b]], sub, topk=cfg.topk, W=cfg.window, cand_block=cfg.cand_block)
        need = np.unique(np.concatenate([d["topk"][0] for d in dry] + [np.zeros(0, np.int64)]))
        need = need[need < n_pre].astype(np.int64)
        tok = torch.as_tensor((r * need[:, None] + np.arange(r)[None]).reshape(-1), device=x.device)
        xs = _host_bits(x[tok])
        ws = None if w is None else _host_bits(w[tok])
        kb = _host_bits(k[:n_pre])
        for i, j in enumerate(need.tolist()):
            oc.write(0, r * j, xs[r * i:r * i + r], None if ws is None else ws[r * i:r * i + r], kb[j:j + 1])
        out[b] = (oc, start, wx, ww, wk, sub)
        del x, w, k
    return out


def cpu_baseline_decode(case, rep, seqs, min_seconds: float, sample_note: str):
    """The oracle's decode step (the step's write, then every layer: selection and
    attention) timed on sampled sequences of the workload, on the host cores."""
    from oracle.schedule import run_decode
    cfg = case.cfg
    specs = [dict(mode=sp.mode, pool_blocks=sp.pool_blocks, q=_host_bits(L["q"]), q_idx=_host_bits(L["q_idx"]),
                  w_idx=_host_bits(L["w_idx"]), swa=_host_bits(L["swa"])) for sp, L in zip(cfg.layers, rep.layers)]
    log(f"cpu baseline {cfg.name}: oracle caches for sequences {list(seqs)} (untimed)")
    caches = _oracle_decode_caches(case, rep, seqs, specs)
    log(f"cpu baseline {cfg.name}: timing the oracle")
    t0 = time.perf_counter()
    done = 0
    while True:
        for b in seqs:
            oc, start, wx, ww, wk, sub = caches[b]
            oc.write(0, start, wx, ww, wk)
            run_decode(oc, [case.ctx_len[b]], sub, topk=cfg.topk, W=cfg.window, cand_block=cfg.cand_block)
            done += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    cores, blas = _host_threads()
    return {"value": round(done / dt, 3), "unit": "queries/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"{sample_note}: sequences {list(seqs)} of {case.B} (lengths "
                      f"{[case.ctx_len[b] for b in seqs]}), {done} queries in {dt:.2f}s; each query is the "
                      f"oracle's whole step for its sequence (the step's write, then {len(cfg.layers)} layers of "
                      f"selection and attention); oracle cache set up untimed; numpy float64, BLAS on "
                      f"{blas} threads, elementwise work on one"}


def cpu_baseline_hisa(case, seqs, layer, keep: int, min_seconds: float):
    """The oracle's HISA selection (block summaries, their top blocks, the top-K
    within them) timed on sampled sequences."""
    from oracle import OracleCache
    from oracle.hisa import hisa_layer
    cfg = case.cfg
    caches = {}
    for b in seqs:
        bt, P = _seq_table(case, b)
        oc = OracleCache(P, bt)
        _, _, k = case.seq_tokens(b)
        oc.write(0, 0, None, None, _host_bits(k), latent=False)
        caches[b] = (oc, _host_bits(layer["q_idx"][b]), _host_bits(layer["w_idx"][b]))
        del k
    t0 = time.perf_counter()
    done = 0
    while True:
        for b in seqs:
            oc, qi, wi = caches[b]
            hisa_layer(oc, 0, case.n_vis[b], qi, wi, cfg.cand_block, keep, cfg.topk)
            done += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    cores, blas = _host_threads()
    return {"value": round(done / dt, 3), "unit": "selections/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle",
            "sample": f"sequences {list(seqs)} of {case.B}, {done} selections in {dt:.2f}s; the oracle recomputes "
                      f"every block summary per selection; oracle keys set up untimed; numpy float64"}


def cpu_baseline_prefill(case, ch, seqs, n_queries: int, sample_note: str):
    """The oracle's chunked prefill, extrapolated from a sample: per sampled sequence the
    chunk's write (2,048 merged entries) is timed whole, and n_queries evenly spaced
    chunk queries (first and last included) are timed; the chunk's time is the write
    plus C times the mean query time.  Untimed set-up: every indexer key, and the
    latent rows the sampled queries read (from a dry run of their selection)."""
    from oracle import OracleCache
    from oracle.indexer import index_scores, topk_select
    from oracle.schedule import n_visible, run_prefill
    cfg = case.cfg
    C = cfg.C
    qs = np.unique(np.linspace(0, C - 1, n_queries).round().astype(int)).tolist()
    q_all, qi_all, wi_all, loc_all = (_host_bits(ch[n]) for n in ("q", "q_idx", "w_idx", "local"))
    t_write = t_query = 0.0
    n_q = 0
    for b in seqs:
        bt, P = _seq_table(case, b, (cfg.prior + C) // 2)
        x, w, k = case.prior_tokens(b)
        xb, wb, kb = _host_bits(x), _host_bits(w), _host_bits(k)
        cx, cw, ck = _host_bits(ch["x"][b]), _host_bits(ch["w"][b]), _host_bits(ch["k_idx"][b])
        oc = OracleCache(P, bt)
        oc.write(0, 0, None, None, kb, latent=False)
        oc.write(0, cfg.prior, None, None, ck, latent=False)
        keys = oc.index_keys(0, np.arange(n_visible(cfg.prior + C - 1)))
        need = set()
        for i in qs:
            nv = n_visible(cfg.prior + i)
            need.update(topk_select(index_scores(qi_all[b, i], wi_all[b, i], keys[:nv]), cfg.topk).tolist())
        need = np.array(sorted(j for j in need if 2 * j < cfg.prior), dtype=np.int64)
        for run in np.split(need, np.nonzero(np.diff(need) != 1)[0] + 1) if need.size else []:
            j0, j1 = int(run[0]), int(run[-1]) + 1
            oc.write(0, 2 * j0, xb[2 * j0:2 * j1], wb[2 * j0:2 * j1], kb[j0:j1])
        del x, w, k, xb, wb
        t0 = time.perf_counter()
        oc.write(0, cfg.prior, cx, cw, ck)                    # the chunk's write path
        t1 = time.perf_counter()
        run_prefill(oc, [cfg.prior], C, q_all[b:b + 1], qi_all[b:b + 1], wi_all[b:b + 1], loc_all[b:b + 1],
                    topk=cfg.topk, W=cfg.window, queries=[(0, i) for i in qs])
        t2 = time.perf_counter()
        t_write += t1 - t0
        t_query += t2 - t1
        n_q += len(qs)
    per_query = t_query / n_q
    per_chunk = t_write / len(seqs) + C * per_query
    cores, blas = _host_threads()
    return {"value": round(C / per_chunk, 3), "unit": "tokens/s", "cores": cores, "blas_threads": blas,
            "kind": "oracle", "extrapolated": True,
            "sample": f"{sample_note}: sequences {list(seqs)} of {case.B}; per sequence the chunk's write "
                      f"({C // 2} entries, timed whole: {t_write / len(seqs):.2f}s) and {len(qs)} evenly spaced "
                      f"chunk queries incl. first and last ({per_query * 1e3:.1f} ms each); the chunk's time is "
                      f"extrapolated as write + {C} x mean query time = {per_chunk:.1f}s; numpy float64"}


if __name__ == "__main__":
    sys.exit(main())
