"""Decode workloads at full size, launched as the benchmark launches them, with the
oracle checking sampled sequences.

The GPU runs the whole batch through the layer schedule (write, Full with the HSI
pool, Reindex, Reuse, attention after every layer).  For each sampled sequence the
oracle stores the indexer keys of every entry, repeats the schedule's selections
itself, stores the latent rows those selections read (the only latent rows the
attention touches), and runs its own decode.  Checks per sampled sequence and
layer: top-K sets and HSI pools up to near-ties (1e-3 of the cut-off score),
attention rows within the 2e-3 bar wherever the GPU's selection equals the
oracle's, and whole-batch properties (sizes, order, visibility) for every sequence.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import OracleCache
from oracle.indexer import full_layer, index_scores, pool_positions, reindex_layer
from oracle.schedule import run_decode
from synth import CONFIGS, make_decode_case
from tests.helpers import bits, check_attention_rows, check_topk_set

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _build_and_run(cfg_id, pick):
    import fp4_kv_cache_write_amd as fk
    cfg = CONFIGS[cfg_id]
    case = make_decode_case(cfg, DEV)
    seqs = pick(case)
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device=DEV)
    bt = case.block_table.to(DEV)
    tokens = {}
    for b in range(case.B):
        x, w, k = case.seq_tokens(b)
        sub = fk.PagedCache(gc.lat_codes, gc.lat_scales, gc.idx_codes, gc.idx_scales, bt[b:b + 1].contiguous())
        fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device=DEV), x[None].contiguous(), w[None].contiguous(),
                    k[None].contiguous())
        if b in seqs:
            tokens[b] = [x.cpu(), w.cpu(), k.cpu()]
        del x, w, k
    if cfg.append > 0:
        xa, wa, ka, start = case.append_tokens()
        fk.write_kv(gc, start.to(DEV), xa, wa, ka)
        for b in seqs:
            tokens[b] = [torch.cat([tokens[b][0], xa[b].cpu()]), torch.cat([tokens[b][1], wa[b].cpu()]),
                         torch.cat([tokens[b][2], ka[b].cpu()])]
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
        o, _ = fk.sparse_decode(gc, ctx, L["q"], tk, L["swa"])
        res.append(dict(topk=tk.cpu().numpy(), pool=None if pool is None else pool.cpu().numpy(), o=bits(o)))
    torch.cuda.synchronize()
    return case, seqs, tokens, res


def _oracle(case, seqs, tokens):
    cfg = case.cfg
    oc = OracleCache(case.n_pages, case.block_table.numpy())
    specs = []
    for l, spec in enumerate(cfg.layers):
        L = case.layer(l)
        specs.append(dict(mode=spec.mode, pool_blocks=spec.pool_blocks, q=bits(L["q"]), q_idx=bits(L["q_idx"]),
                          w_idx=bits(L["w_idx"]), swa=bits(L["swa"])))
    for b in seqs:
        x, w, k = (bits(t) for t in tokens[b])
        oc.write(b, 0, x, w, k, latent=False)
        # the schedule's selections, to know which latent rows the attention reads
        nv = case.ctx_len[b] // 2
        need, cur, blocks = set(), None, np.zeros(0, np.int64)
        for sp in specs:
            if sp["mode"] == "full":
                cur, bl, _ = full_layer(oc, b, nv, sp["q_idx"][b], sp["w_idx"][b], cfg.topk, sp["pool_blocks"],
                                        cfg.cand_block)
                if sp["pool_blocks"] > 0:
                    blocks = bl
            elif sp["mode"] == "reindex":
                cur, _ = reindex_layer(oc, b, nv, sp["q_idx"][b], sp["w_idx"][b], blocks, cfg.cand_block, cfg.topk)
            need.update(np.asarray(cur).tolist())
        for j in sorted(need):
            oc.write(b, 2 * j, x[2 * j:2 * j + 2], w[2 * j:2 * j + 2], k[j:j + 1])
    ref = run_decode(oc, case.ctx_len, specs, topk=cfg.topk, W=cfg.window, cand_block=cfg.cand_block, seqs=seqs)
    return oc, specs, ref


def _block_scores(s, nv, cb):
    nb = (nv + cb - 1) // cb
    pad = np.full(nb * cb, -np.inf)
    pad[:nv] = s
    beta = pad.reshape(nb, cb).max(axis=1)
    beta[(nv - 1) // cb] = np.inf
    return beta


def _check(case, seqs, res, oc, specs, ref, min_frac=0.7):
    cfg = case.cfg
    compared = total = 0
    worst = 0.0
    for b in seqs:
        nv = case.ctx_len[b] // 2
        pool_same = True
        for l, sp in enumerate(specs):
            g_tk = res[l]["topk"][b]
            if sp["mode"] == "full":
                s = index_scores(sp["q_idx"][b], sp["w_idx"][b], oc.index_keys(b, np.arange(nv)))
                check_topk_set(g_tk, np.arange(nv), s, cfg.topk)
                if sp["pool_blocks"] > 0:
                    g_pool = res[l]["pool"][b]
                    beta = _block_scores(s, nv, cfg.cand_block)
                    check_topk_set(g_pool, np.arange(len(beta)), beta, sp["pool_blocks"])
                    pool_same = np.array_equal(g_pool[g_pool >= 0], ref[l]["pool"][b])
            elif sp["mode"] == "reindex" and pool_same:
                pos = pool_positions(ref[l]["pool"][b], nv, cfg.cand_block)
                s2 = index_scores(sp["q_idx"][b], sp["w_idx"][b], oc.index_keys(b, pos))
                check_topk_set(g_tk, pos, s2, cfg.topk)
            total += 1
            if np.array_equal(g_tk[g_tk >= 0], ref[l]["topk"][b]):
                worst = max(worst, check_attention_rows(res[l]["o"][b], ref[l]["o"][b]))
                compared += 1
    assert compared >= min_frac * total, f"only {compared}/{total} selections identical"
    return compared, total, worst


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


def test_config1_b32_ctx64k_three_layers():
    case, seqs, tokens, res = _build_and_run(1, lambda c: (0, 13, 31))
    oc, specs, ref = _oracle(case, seqs, tokens)
    compared, total, worst = _check(case, seqs, res, oc, specs, ref)
    _batch_properties(case, res)
    print(f"config 1: {compared}/{total} layer outputs compared, worst {worst / 2e-3:.4f} of the bar")


def test_config2_b8_ctx1m_full_scan():
    case, seqs, tokens, res = _build_and_run(2, lambda c: (5,))
    oc, specs, ref = _oracle(case, seqs, tokens)
    compared, total, worst = _check(case, seqs, res, oc, specs, ref, min_frac=1.0)
    _batch_properties(case, res)
    print(f"config 2: {compared}/{total} layer outputs compared, worst {worst / 2e-3:.4f} of the bar")


def test_config4_b128_mixed_lengths_four_layers():
    def pick(c):
        L = np.asarray(c.ctx_len)
        return (int(L.argmin()), int(L.argmax()), 77)

    case, seqs, tokens, res = _build_and_run(4, pick)
    oc, specs, ref = _oracle(case, seqs, tokens)
    compared, total, worst = _check(case, seqs, res, oc, specs, ref)
    _batch_properties(case, res)
    print(f"config 4: {compared}/{total} layer outputs compared, worst {worst / 2e-3:.4f} of the bar "
          f"(lengths {[case.ctx_len[b] for b in seqs]})")
