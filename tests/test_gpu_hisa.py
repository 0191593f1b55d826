"""GPU parity of the HISA block-mean pool: block summaries bit-exact against the
oracle (all blocks, and the newest block refreshed after an append), the two-stage
selection against the oracle's scores, and the one-entry-block reduction to Full."""
import numpy as np
import pytest
import torch

from oracle import block_summaries, index_scores, pack_nibbles
from oracle.hisa import hisa_layer
from oracle.indexer import pool_positions
from synth import make_decode_case, small_decode
from tests.helpers import bits, check_topk_set, gpu_cache_for, oracle_cache_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    return m


def _block_cache(fk, B, max_ctx, cb, ratio=2):
    """Ratio-1 cache with one slot per block: sequence b owns pages b*P .. b*P+P-1."""
    nb = -(-(max_ctx // ratio) // cb)
    P = max(1, -(-nb // 64))
    bt = torch.arange(B * P, dtype=torch.int32).reshape(B, P)
    return fk.PagedCache.allocate(B * P, bt, ratio=1), nb


def _check_blocks(blocks, oc, case, cb):
    bi = blocks.idx_codes.cpu().numpy()
    bs = blocks.idx_scales.cpu().numpy()
    bt = blocks.block_table.cpu().numpy()
    for b in range(case.B):
        codes, scales = block_summaries(oc, b, case.n_vis[b], cb)
        ks = np.arange(codes.shape[0])
        pg, sl = bt[b, ks // 64], ks % 64
        assert np.array_equal(bi[pg, sl], pack_nibbles(codes)), f"seq {b}: block codes"
        assert np.array_equal(bs[pg, sl], scales), f"seq {b}: block scales"


@pytest.mark.parametrize("cb", [8, 4, 32])
def test_block_summaries_match_oracle_bytes(fk, cb):
    ctx = (20000, 2, 1030, 65536)
    cfg = small_decode(1, B=len(ctx), ctx=ctx, pages="random", heavy_frac=0.05, append=0, seed=1301 + cb)
    case = make_decode_case(cfg, "cpu")
    oc, gc = oracle_cache_for(case), gpu_cache_for(case)
    blocks, _ = _block_cache(fk, case.B, max(ctx), cb)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    nb = fk.block_keys(gc, blocks, ctx_len, max(ctx), cand_block=cb)
    torch.cuda.synchronize()
    assert nb.cpu().tolist() == [-(-v // cb) for v in case.n_vis]
    _check_blocks(blocks, oc, case, cb)


def test_newest_block_refresh_after_append(fk):
    # Decode keeps finished blocks and refreshes only the blocks the new entries fall
    # in: summarise the pre-built entries, append 64 tokens (32 entries), refresh from
    # the block that held the last old entry, and every block equals the oracle's
    # summary of the whole cache.
    cb = 8
    cfg = small_decode(4, B=3, ctx=(700, 4000, 130), pages="random", append=64, seed=1311)
    case = make_decode_case(cfg, "cpu")
    oc, gc = oracle_cache_for(case), gpu_cache_for(case)          # the pre-built entries
    max_ctx = max(case.ctx_len)
    blocks, _ = _block_cache(fk, case.B, max_ctx, cb)
    before = torch.tensor(case.prebuilt, dtype=torch.int32, device="cuda")
    fk.block_keys(gc, blocks, before, max_ctx, cand_block=cb)
    x, w, k, start = case.append_tokens()
    for b in range(case.B):
        oc.write(b, int(start[b]), bits(x[b]), bits(w[b]), bits(k[b]))
    fk.write_kv(gc, start.cuda(), x.cuda(), w.cuda(), k.cuda())
    first = torch.tensor([max(0, (P // 2 - 1) // cb) for P in case.prebuilt], dtype=torch.int32, device="cuda")
    after = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    fk.block_keys(gc, blocks, after, max_ctx, cand_block=cb, blk_first=first, n_span=32 // cb + 1)
    torch.cuda.synchronize()
    _check_blocks(blocks, oc, case, cb)


@pytest.mark.parametrize("cb,keep,topk", [(8, 300, 512), (4, 100, 64), (16, 512, 512)])
def test_hisa_selection_matches_oracle(fk, cb, keep, topk):
    ctx = (65536, 9000, 800)
    cfg = small_decode(1, B=len(ctx), ctx=ctx, pages="random", heavy_frac=0.05, append=0, seed=1321 + cb)
    case = make_decode_case(cfg, "cpu")
    oc, gc = oracle_cache_for(case), gpu_cache_for(case)
    blocks, max_blocks = _block_cache(fk, case.B, max(ctx), cb)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    nb = fk.block_keys(gc, blocks, ctx_len, max(ctx), cand_block=cb)
    L = case.layer(0)
    tk, pool = fk.index_hisa(gc, blocks, nb, max_blocks, ctx_len, L["q_idx"].cuda(), L["w_idx"].cuda(),
                             keep_blocks=keep, topk=topk, cand_block=cb)
    torch.cuda.synchronize()
    tk, pool = tk.cpu().numpy(), pool.cpu().numpy()
    for b in range(case.B):
        n_vis = case.n_vis[b]
        _, _, S = hisa_layer(oc, b, n_vis, bits(L["q_idx"][b]), bits(L["w_idx"][b]), cb, keep, topk)
        check_topk_set(pool[b], np.arange(len(S)), S, keep)                # stage 1 over the block summaries
        pos = pool_positions(pool[b][pool[b] >= 0], n_vis, cb)
        s = index_scores(bits(L["q_idx"][b]), bits(L["w_idx"][b]), oc.index_keys(b, pos))
        check_topk_set(tk[b], pos, s, topk)                                # stage 2 inside the GPU's pool


def test_one_entry_blocks_reproduce_the_full_top_k(fk):
    # Block keys of single entries carry the entries' key values, so stage 1 scores
    # them exactly as the Full scan does and a pool of >= K blocks holds the Full top-K.
    ctx = (30000, 5000)
    cfg = small_decode(1, B=2, ctx=ctx, pages="random", heavy_frac=0.05, append=0, seed=1331)
    case = make_decode_case(cfg, "cpu")
    gc = gpu_cache_for(case)
    blocks, max_blocks = _block_cache(fk, case.B, max(ctx), 1)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    nb = fk.block_keys(gc, blocks, ctx_len, max(ctx), cand_block=1)
    L = case.layer(0)
    q, w = L["q_idx"].cuda(), L["w_idx"].cuda()
    tk, _ = fk.index_hisa(gc, blocks, nb, max_blocks, ctx_len, q, w, keep_blocks=1024, topk=512, cand_block=1)
    full, _ = fk.index_full(gc, ctx_len, max(ctx), q, w, topk=512)
    torch.cuda.synchronize()
    assert torch.equal(tk.cpu(), full.cpu())


def test_hisa_at_full_size_on_sampled_sequences(fk):
    # The headline shape (32 sequences x 65,536 tokens, 5% heavy-tailed keys): every
    # block summary of the sampled sequences is bit-exact, and both selection stages
    # agree with the oracle's scores; the whole batch is launched as one call.
    from oracle import OracleCache
    from synth import CONFIGS
    cfg = CONFIGS[1]
    cb, keep, topk = cfg.cand_block, 512, cfg.topk
    case = make_decode_case(cfg, "cuda")
    seqs = (0, 17, 31)
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device="cuda")
    bt = case.block_table.to("cuda")
    oc = OracleCache(case.n_pages, case.block_table.numpy())
    for b in range(case.B):
        x, w, k = case.seq_tokens(b)
        sub = fk.PagedCache(gc.lat_codes, gc.lat_scales, gc.idx_codes, gc.idx_scales, bt[b:b + 1].contiguous())
        fk.write_kv(sub, torch.zeros(1, dtype=torch.int32, device="cuda"), x[None].contiguous(), w[None].contiguous(),
                    k[None].contiguous())
        if b in seqs:
            oc.write(b, 0, None, None, bits(k), latent=False)
        del x, w, k
    max_ctx = max(case.ctx_len)
    blocks, max_blocks = _block_cache(fk, case.B, max_ctx, cb)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    nb = fk.block_keys(gc, blocks, ctx_len, max_ctx, cand_block=cb)
    L = case.layer(0)
    tk, pool = fk.index_hisa(gc, blocks, nb, max_blocks, ctx_len, L["q_idx"], L["w_idx"], keep_blocks=keep,
                             topk=topk, cand_block=cb)
    torch.cuda.synchronize()
    bi, bs = blocks.idx_codes.cpu().numpy(), blocks.idx_scales.cpu().numpy()
    btb = blocks.block_table.cpu().numpy()
    tk, pool = tk.cpu().numpy(), pool.cpu().numpy()
    for b in seqs:
        n_vis = case.n_vis[b]
        codes, scales = block_summaries(oc, b, n_vis, cb)
        ks = np.arange(codes.shape[0])
        assert np.array_equal(bi[btb[b, ks // 64], ks % 64], pack_nibbles(codes)), f"seq {b}: block codes"
        assert np.array_equal(bs[btb[b, ks // 64], ks % 64], scales), f"seq {b}: block scales"
        q, w = bits(L["q_idx"][b]), bits(L["w_idx"][b])
        _, _, S = hisa_layer(oc, b, n_vis, q, w, cb, keep, topk)
        check_topk_set(pool[b], np.arange(len(S)), S, keep)
        pos = pool_positions(pool[b][pool[b] >= 0], n_vis, cb)
        check_topk_set(tk[b], pos, index_scores(q, w, oc.index_keys(b, pos)), topk)
    assert np.all((tk >= -1) & (tk < max(case.n_vis)))
