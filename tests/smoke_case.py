"""One small CSA2 decode step on cuda:0, checked against the CPU oracle.

Write path (pre-built cache + a 2-token pair completing the newest entry), Full
layer with HSI pool, attention, Reindex layer, attention, Reuse layer, attention.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.indexer import index_scores, pool_positions
from oracle.schedule import run_decode
from synth import LayerSpec, make_decode_case, small_decode
from tests.helpers import (AttentionReport, bits, cache_bytes_equal, check_pool_set, check_topk_set,
                           oracle_cache_for)


def run_smoke() -> None:
    import fp4_kv_cache_write_amd as fk
    fk.lib()
    if not torch.cuda.is_available():
        raise RuntimeError("smoke needs a GPU")
    dev = "cuda:0"
    topk, pool_blocks, cb, W = 128, 40, 8, 128
    cfg = small_decode(1, B=2, ctx=(4096, 1030), H=16, pages="random", append=2, topk=topk,
                       layers=(LayerSpec("full", pool_blocks), LayerSpec("reindex"), LayerSpec("reuse")))
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case)
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device=dev)
    # pre-built tokens, then the step's pair write
    bt = case.block_table.to(dev)
    for b in range(case.B):
        x, w, k = case.seq_tokens(b)
        sub = fk.PagedCache(gc.lat_codes, gc.lat_scales, gc.idx_codes, gc.idx_scales, bt[b:b + 1].contiguous())
        fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device=dev), x.to(dev)[None].contiguous(),
                    w.to(dev)[None].contiguous(), k.to(dev)[None].contiguous())
    xa, wa, ka, start = case.append_tokens()
    fk.write_kv(gc, start.to(dev), xa.to(dev), wa.to(dev), ka.to(dev))
    for b in range(case.B):
        oc.write(b, int(start[b]), bits(xa[b]), bits(wa[b]), bits(ka[b]))
    torch.cuda.synchronize()
    diff = cache_bytes_equal(gc, oc)
    assert all(v == 0 for v in diff.values()), f"cache bytes differ: {diff}"

    ctx = torch.tensor(case.ctx_len, dtype=torch.int32, device=dev)
    L = [case.layer(l) for l in range(3)]
    tk, pool = fk.index_full(gc, ctx, max(case.ctx_len), L[0]["q_idx"].to(dev), L[0]["w_idx"].to(dev), topk=topk,
                             pool_blocks=pool_blocks, cand_block=cb)
    o0, l0 = fk.sparse_decode(gc, ctx, L[0]["q"].to(dev), tk, L[0]["swa"].to(dev))
    tk2 = fk.reindex(gc, ctx, L[1]["q_idx"].to(dev), L[1]["w_idx"].to(dev), pool, topk=topk, cand_block=cb)
    o1, l1 = fk.sparse_decode(gc, ctx, L[1]["q"].to(dev), tk2, L[1]["swa"].to(dev))
    o2, l2 = fk.sparse_decode(gc, ctx, L[2]["q"].to(dev), tk2, L[2]["swa"].to(dev))
    torch.cuda.synchronize()
    tk, pool, tk2 = tk.cpu().numpy(), pool.cpu().numpy(), tk2.cpu().numpy()
    outs = [bits(o.cpu()) for o in (o0, o1, o2)]
    lses = [x.cpu().numpy() for x in (l0, l1, l2)]
    gsel = [tk, tk2, tk2]
    # the oracle runs the same three layers on its own cache; its attention reads the
    # GPU's selections (a set that differs only by near-tied scores is as correct)
    specs = [dict(mode=sp.mode, pool_blocks=sp.pool_blocks, q=bits(L[l]["q"]), q_idx=bits(L[l]["q_idx"]),
                  w_idx=bits(L[l]["w_idx"]), swa=bits(L[l]["swa"])) for l, sp in enumerate(cfg.layers)]
    attend = [{b: gsel[l][b][gsel[l][b] >= 0] for b in range(case.B)} for l in range(3)]
    ref = run_decode(oc, case.ctx_len, specs, topk=topk, W=W, cand_block=cb, attend_on=attend)
    rep, same = AttentionReport(), 0
    for b in range(case.B):
        nv = case.n_vis[b]
        s = index_scores(specs[0]["q_idx"][b], specs[0]["w_idx"][b], oc.index_keys(b, np.arange(nv)))
        check_topk_set(tk[b], np.arange(nv), s, topk)
        check_pool_set(pool[b], s, nv, cb, pool_blocks)
        pos = pool_positions(pool[b][pool[b] >= 0], nv, cb)
        s2 = index_scores(specs[1]["q_idx"][b], specs[1]["w_idx"][b], oc.index_keys(b, pos))
        check_topk_set(tk2[b], pos, s2, topk)
        for l in range(3):
            rep.check(outs[l][b], ref[l]["o"][b], lses[l][b], ref[l]["lse"][b])
            same += int(np.array_equal(attend[l][b], ref[l]["topk"][b]))
    assert rep.n == 6
    print(f"smoke ok: write bit-exact, top-K/pool/reindex match, attention {rep}; "
          f"{same}/6 selections identical to the oracle's")


if __name__ == "__main__":
    run_smoke()
