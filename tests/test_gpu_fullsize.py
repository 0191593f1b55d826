"""Decode workloads at full size, launched as the benchmark launches them, with the
oracle checking sampled sequences.

The GPU runs the whole batch through the layer schedule (write, Full with the HSI
pool, Reindex, Reuse, attention after every layer).  For each sampled sequence the
oracle stores the indexer keys of every entry and the latent rows of the entries the
GPU selected (regenerated from the seeded inputs), then checks every layer:
- Full: the GPU's top-K set and HSI pool against the oracle's scores, up to
  near-ties (1e-3 of the cut-off score);
- Reindex: the GPU's top-K against the oracle's scores over the GPU's own pool;
- Reuse: the previous layer's selection, unchanged;
- attention, always: the oracle's decode on the GPU's own selection (a set that
  differs by near-ties is as correct), within the 2e-3 bar, lse within 1e-4.
Whole-batch properties (sizes, order, visibility, finite outputs) hold for every
sequence.  The summary line also counts how many selections equal the oracle's.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import OracleCache
from oracle.indexer import index_scores, pool_positions
from oracle.schedule import run_decode
from synth import CONFIGS, make_decode_case
from tests.helpers import AttentionReport, bits, check_pool_set, check_topk_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _build_and_run(cfg_id, pick):
    import fp4_kv_cache_write_amd as fk
    cfg = CONFIGS[cfg_id]
    case = make_decode_case(cfg, DEV)
    seqs = pick(case)
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device=DEV)
    bt = case.block_table.to(DEV)
    keys = {}
    for b in range(case.B):
        x, w, k = case.seq_tokens(b)
        sub = fk.PagedCache(gc.lat_codes, gc.lat_scales, gc.idx_codes, gc.idx_scales, bt[b:b + 1].contiguous())
        fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device=DEV), x[None].contiguous(), w[None].contiguous(),
                    k[None].contiguous())
        if b in seqs:
            keys[b] = k.cpu()
        del x, w, k
    if cfg.append > 0:
        xa, wa, ka, start = case.append_tokens()
        fk.write_kv(gc, start.to(DEV), xa, wa, ka)
        for b in seqs:
            keys[b] = torch.cat([keys[b], ka[b].cpu()])
    ctx = torch.tensor(case.ctx_len, dtype=torch.int32, device=DEV)
    max_ctx = max(case.ctx_len)
    res = []
    tk, pool = None, None
    for l, spec in enumerate(cfg.layers):
        L = case.layer(l)
        if spec.mode == "full":
            tk, p = fk.index_full(gc, ctx, max_ctx, L["q_idx"], L["w_idx"], topk=cfg.topk,
                                  pool_blocks=spec.pool_blocks, cand_block=cfg.cand_block)
            if spec.pool_blocks > 0:
                pool = p
        elif spec.mode == "reindex":
            tk = fk.reindex(gc, ctx, L["q_idx"], L["w_idx"], pool, topk=cfg.topk, cand_block=cfg.cand_block)
        o, lse = fk.sparse_decode(gc, ctx, L["q"], tk, L["swa"])
        res.append(dict(topk=tk.cpu().numpy(), pool=None if pool is None else pool.cpu().numpy(), o=bits(o),
                        lse=lse.cpu().numpy()))
    torch.cuda.synchronize()
    return case, seqs, keys, res


def _entry_tokens(case, b, js):
    """Write inputs (x, w bits) of the token pairs merged into entries js of sequence b,
    regenerated from the seeded recipe (pre-built tokens, then the step's append)."""
    x, w, _ = case.seq_tokens(b)
    if case.cfg.append > 0:
        xa, wa, _, _ = case.append_tokens()
        x = torch.cat([x, xa[b].to(x.device)])
        w = torch.cat([w, wa[b].to(w.device)])
    tok = torch.as_tensor(np.stack([2 * js, 2 * js + 1], axis=1).reshape(-1), device=x.device)
    return bits(x[tok]), bits(w[tok])


def _oracle(case, seqs, keys, res):
    cfg = case.cfg
    oc = OracleCache(case.n_pages, case.block_table.numpy())
    specs = []
    for l, spec in enumerate(cfg.layers):
        L = case.layer(l)
        specs.append(dict(mode=spec.mode, pool_blocks=spec.pool_blocks, q=bits(L["q"]), q_idx=bits(L["q_idx"]),
                          w_idx=bits(L["w_idx"]), swa=bits(L["swa"])))
    attend = [dict() for _ in specs]
    for b in seqs:
        kb = bits(keys[b])
        oc.write(b, 0, None, None, kb, latent=False)
        sels = [r["topk"][b][r["topk"][b] >= 0].astype(np.int64) for r in res]
        for l, sel in enumerate(sels):
            attend[l][b] = sel
        need = np.unique(np.concatenate(sels))
        xr, wr = _entry_tokens(case, b, need)
        for i, j in enumerate(need):
            oc.write(b, 2 * int(j), xr[2 * i:2 * i + 2], wr[2 * i:2 * i + 2], kb[j:j + 1])
    ref = run_decode(oc, case.ctx_len, specs, topk=cfg.topk, W=cfg.window, cand_block=cfg.cand_block, seqs=seqs,
                     attend_on=attend)
    return oc, specs, ref


def _check(case, seqs, res, oc, specs, ref):
    cfg = case.cfg
    rep = AttentionReport()
    same = total = 0
    for b in seqs:
        nv = case.ctx_len[b] // 2
        g_pool = None
        for l, sp in enumerate(specs):
            g_tk = res[l]["topk"][b]
            if sp["mode"] == "full":
                s = index_scores(sp["q_idx"][b], sp["w_idx"][b], oc.index_keys(b, np.arange(nv)))
                check_topk_set(g_tk, np.arange(nv), s, cfg.topk)
                if sp["pool_blocks"] > 0:
                    p = res[l]["pool"][b]
                    check_pool_set(p, s, nv, cfg.cand_block, sp["pool_blocks"])
                    g_pool = p[p >= 0]
            elif sp["mode"] == "reindex":
                pos = pool_positions(g_pool, nv, cfg.cand_block)
                s2 = index_scores(sp["q_idx"][b], sp["w_idx"][b], oc.index_keys(b, pos))
                check_topk_set(g_tk, pos, s2, cfg.topk)
            else:
                assert np.array_equal(g_tk, res[l - 1]["topk"][b]), "Reuse changed the selection"
            rep.check(res[l]["o"][b], ref[l]["o"][b], res[l]["lse"][b], ref[l]["lse"][b])
            same += int(np.array_equal(g_tk[g_tk >= 0], ref[l]["topk"][b]))
            total += 1
    assert rep.n == total == len(seqs) * len(specs)
    return rep, same, total


def _batch_properties(case, res):
    cfg = case.cfg
    nv = np.asarray(case.ctx_len) // 2
    for l, r in enumerate(res):
        tk = r["topk"]
        valid = tk >= 0
        if cfg.layers[l].mode == "full":
            assert np.all(valid.sum(-1) == np.minimum(nv, cfg.topk))
        assert np.all(np.where(valid, tk, -1) < nv[:, None])
        filler = np.iinfo(np.int32).max // 2 + np.arange(tk.shape[1])
        assert np.all(np.diff(np.where(valid, tk, filler), axis=-1) > 0)
        assert not np.any((r["o"] & 0x7f80) == 0x7f80), "inf or NaN in the attention output"
        assert np.all(np.isfinite(r["lse"]))


def _run(cfg_id, pick, label):
    case, seqs, keys, res = _build_and_run(cfg_id, pick)
    oc, specs, ref = _oracle(case, seqs, keys, res)
    rep, same, total = _check(case, seqs, res, oc, specs, ref)
    _batch_properties(case, res)
    print(f"{label}: sequences {list(seqs)} (lengths {[case.ctx_len[b] for b in seqs]}); {rep}; "
          f"{same}/{total} selections identical to the oracle's")


def test_config1_b32_ctx64k_three_layers():
    _run(1, lambda c: (0, 4, 9, 13, 18, 22, 27, 31), "config 1")


def test_config2_b8_ctx1m_full_scan():
    _run(2, lambda c: (0, 5), "config 2")


def test_config4_b128_mixed_lengths_four_layers():
    def pick(c):
        L = np.asarray(c.ctx_len)
        lo, hi = int(L.argmin()), int(L.argmax())
        rest = [b for b in np.random.default_rng(404).permutation(c.B).tolist() if b not in (lo, hi)]
        return tuple(sorted([lo, hi] + rest[:6]))

    _run(4, pick, "config 4")
