"""GPU parity of the decoder's ratio-1 cache (one entry per token) against the oracle.

[P1] §2.3.1: the compressor's ratio-1 case keeps the decoder's main KV unmerged;
[P1] §2.3.4: the decoder's Full layer builds an HSI pool of 2048 blocks of 8
positions for its Reindex layers.  The write must be bit-exact; selections match
the oracle's scores up to near-ties; attention meets the 2e-3 bar.
"""
import math

import numpy as np
import pytest
import torch

from oracle import OracleCache, sparse_attention
from oracle.attention import gather_rows
from oracle.indexer import full_layer, index_scores, pool_positions
from synth import CONFIGS, make_decode_case, small_decode
from tests.helpers import (bits, cache_bytes_equal, check_attention_rows, check_topk_set, gpu_cache_for,
                           oracle_cache_for)
from tests.test_gpu_index import _check_pool

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    return m


def _case(ctx, H=16, pool_blocks=2048, pages="random", seed=None):
    cfg = small_decode(5, B=len(ctx), ctx=ctx, H=H, pages=pages, heavy_frac=0.05, append=0, seed=seed)
    assert cfg.ratio == 1 and cfg.layers[0].pool_blocks == pool_blocks
    return make_decode_case(cfg, "cpu")


def test_ratio1_write_is_bit_exact(fk):
    # pre-built tokens (one entry each), then a 5-token append at an odd position
    case = _case((3001, 130, 64))
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    assert all(v == 0 for v in cache_bytes_equal(gc, oc).values())
    g = torch.Generator().manual_seed(7)
    x = torch.randn(case.B, 5, 512, generator=g).to(torch.bfloat16)
    k = torch.randn(case.B, 5, 64, generator=g).to(torch.bfloat16)
    start = [37, 125, 59]                                   # odd and even starts, within the pages
    fk.write_kv(gc, torch.tensor(start, dtype=torch.int32, device="cuda"), x.cuda(), None, k.cuda())
    torch.cuda.synchronize()
    for b in range(case.B):
        oc.write(b, start[b], bits(x[b]), None, bits(k[b]))
    assert all(v == 0 for v in cache_bytes_equal(gc, oc).values())


def test_ratio1_full_pool2048_and_reindex(fk):
    # 20000 and 17000 tokens = entries: 2500 and 2125 blocks, so the 2048-block pool
    # is a real cut; 300 tokens: every block is pooled
    case = _case((20000, 17000, 300))
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    L0, L1 = case.layer(0), case.layer(1)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    tk, pool = fk.index_full(gc, ctx_len, max(case.ctx_len), L0["q_idx"].cuda(), L0["w_idx"].cuda(), topk=512,
                             pool_blocks=2048, cand_block=8)
    tk2 = fk.reindex(gc, ctx_len, L1["q_idx"].cuda(), L1["w_idx"].cuda(), pool, topk=512, cand_block=8)
    torch.cuda.synchronize()
    tk, pool, tk2 = tk.cpu().numpy(), pool.cpu().numpy(), tk2.cpu().numpy()
    for b in range(case.B):
        n_vis = case.n_vis[b]
        assert n_vis == case.ctx_len[b]                     # one entry per token
        s = index_scores(bits(L0["q_idx"][b]), bits(L0["w_idx"][b]), oc.index_keys(b, np.arange(n_vis)))
        check_topk_set(tk[b], np.arange(n_vis), s, 512)
        _check_pool(pool[b], s, n_vis, 8, 2048)
        # Reindex over the GPU's own pool, scored by the oracle
        blocks = pool[b][pool[b] >= 0]
        pos = pool_positions(blocks, n_vis, 8)
        s1 = index_scores(bits(L1["q_idx"][b]), bits(L1["w_idx"][b]), oc.index_keys(b, pos))
        check_topk_set(tk2[b], pos, s1, 512)


@pytest.mark.parametrize("split", [True, False], ids=["split", "whole"])
def test_ratio1_attention(fk, split):
    # the newest entry (the current token) is visible at ratio 1 and must be attended
    case = _case((20000, 300, 5001), H=64)
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    L = case.layer(0)
    tk = np.full((case.B, 512), -1, np.int32)
    for b in range(case.B):
        t, _, _ = full_layer(oc, b, case.n_vis[b], bits(L["q_idx"][b]), bits(L["w_idx"][b]), 512)
        tk[b, :len(t)] = t
        tk[b, 0] = case.n_vis[b] - 1 if case.n_vis[b] - 1 not in t else tk[b, 0]
        tk[b] = np.sort(np.where(tk[b] >= 0, tk[b], np.iinfo(np.int32).max))
        tk[b][tk[b] == np.iinfo(np.int32).max] = -1
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    ws = None if split else torch.empty(0, dtype=torch.uint8, device="cuda")
    out, lse = fk.sparse_decode(gc, ctx_len, L["q"].cuda(), torch.from_numpy(tk).cuda(), L["swa"].cuda(), ws=ws)
    torch.cuda.synchronize()
    out_b, lse = bits(out.cpu()), lse.cpu().numpy()
    for b in range(case.B):
        t = case.ctx_len[b] - 1
        ids = tk[b][tk[b] >= 0]
        assert t in ids.tolist()                            # entry t (token t itself) is selectable
        rows = gather_rows(oc, b, ids, bits(L["swa"][b]), t, case.cfg.window)
        o_ref, lse_ref = sparse_attention(bits(L["q"][b]), rows, 1 / math.sqrt(512))
        check_attention_rows(out_b[b], o_ref)
        assert np.allclose(lse[b], lse_ref, rtol=0, atol=1e-4)


def test_ratio1_decoder_full_size_sampled(fk):
    # the decoder workload at its full size (32 x 32K tokens, pool 2048 x 8), sampled:
    # sequences 0 and 31 checked against the oracle for all three layers
    cfg = CONFIGS[5]
    case = make_decode_case(cfg, "cuda")
    gc = gpu_cache_for(case)
    seqs = (0, 31)
    oc = OracleCache(case.n_pages, case.block_table.numpy(), ratio=1)
    for b in seqs:
        x, _, k = case.seq_tokens(b)
        oc.write(b, 0, bits(x), None, bits(k))
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    L0, L1, L2 = case.layer(0), case.layer(1), case.layer(2)
    tk0, pool = fk.index_full(gc, ctx_len, max(case.ctx_len), L0["q_idx"], L0["w_idx"], topk=512,
                              pool_blocks=2048, cand_block=8)
    tk1 = fk.reindex(gc, ctx_len, L1["q_idx"], L1["w_idx"], pool, topk=512, cand_block=8)
    outs = [fk.sparse_decode(gc, ctx_len, L["q"], t, L["swa"])[0] for L, t in ((L0, tk0), (L1, tk1), (L2, tk1))]
    torch.cuda.synchronize()
    tk0, tk1, pool = tk0.cpu().numpy(), tk1.cpu().numpy(), pool.cpu().numpy()
    for b in seqs:
        n_vis = case.n_vis[b]
        s = index_scores(bits(L0["q_idx"][b]), bits(L0["w_idx"][b]), oc.index_keys(b, np.arange(n_vis)))
        check_topk_set(tk0[b], np.arange(n_vis), s, 512)
        _check_pool(pool[b], s, n_vis, 8, 2048)
        pos = pool_positions(pool[b][pool[b] >= 0], n_vis, 8)
        s1 = index_scores(bits(L1["q_idx"][b]), bits(L1["w_idx"][b]), oc.index_keys(b, pos))
        check_topk_set(tk1[b], pos, s1, 512)
        t = case.ctx_len[b] - 1
        for L, ids, o in ((L0, tk0[b], outs[0]), (L1, tk1[b], outs[1]), (L2, tk1[b], outs[2])):
            rows = gather_rows(oc, b, ids[ids >= 0], bits(L["swa"][b]), t, cfg.window)
            o_ref, _ = sparse_attention(bits(L["q"][b]), rows, 1 / math.sqrt(512))
            check_attention_rows(bits(o[b].cpu()), o_ref)
