"""GPU parity of the Full indexer (top-K + HSI pool) and Reindex against the oracle."""
import numpy as np
import pytest
import torch

from oracle.indexer import full_layer, hsi_pool, index_scores, pool_positions, reindex_layer
from synth import make_decode_case, small_decode
from tests.helpers import bits, check_topk_set, gpu_cache_for, oracle_cache_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    return m


def _check_pool(gpu_pool, s, n_vis, cb, nb, tol=1e-3):
    g = np.asarray(gpu_pool)
    valid = g[g >= 0]
    assert np.all(g[len(valid):] == -1) and np.all(np.diff(valid) > 0)
    want, _ = hsi_pool(s, n_vis, cb, nb)
    assert len(valid) == len(want)
    if n_vis == 0:
        return
    latest = (n_vis - 1) // cb
    assert latest in valid.tolist()
    pad = (-n_vis) % cb
    bmax = np.concatenate([s, np.full(pad, -np.inf)]).reshape(-1, cb).max(axis=1)
    bmax[latest] = np.inf
    diff = set(want.tolist()).symmetric_difference(valid.tolist())
    if diff:
        order = np.lexsort((np.arange(len(bmax)), -bmax))
        edge = bmax[order[len(want) - 1]]
        far = [k for k in diff if abs(bmax[k] - edge) > tol]
        assert not far, far


CASES = [
    # (ctx per sequence, topk, pool_blocks, cand_block, pages)
    ((2048,), 512, 256, 8, "identity"),                                   # config-0 shape
    ((0, 2, 14, 1022, 1024, 1026, 8192, 8194, 20000), 512, 40, 8, "random"),  # ragged tails
    ((9000, 30000), 64, 100, 4, "fragmented"),
    ((65536, 3000), 512, 512, 8, "random"),                               # config-1 length
    ((5000,), 2048, 300, 16, "identity"),
    ((16390,), 100, 5, 1, "random"),
    # 133,000 entries at K = 2048: 16384-entry chunks, the chunk groups' pre-merge, and a
    # final merge of 32 keys per thread; the shorter sequence leaves four of five groups empty
    ((266000, 40002), 2048, 64, 8, "random"),
    # 65 sequences: a 5-chunk grid of 325 scan workgroups (the 8-wave scan workgroup),
    # with short and empty sequences whose chunks hold nothing
    (tuple([35000] + [2 * ((i * 97) % 1500) for i in range(64)]), 512, 64, 8, "random"),
]


@pytest.mark.parametrize("ctx,topk,pool_blocks,cb,pages", CASES)
def test_index_full_matches_oracle(fk, ctx, topk, pool_blocks, cb, pages):
    cfg = small_decode(1, B=len(ctx), ctx=ctx, pages=pages, heavy_frac=0.05, append=0,
                       layers=small_decode(1, B=1, ctx=(2,)).layers)
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    L = case.layer(0)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    max_ctx = max(case.ctx_len)
    tk, pool = fk.index_full(gc, ctx_len, max_ctx, L["q_idx"].cuda(), L["w_idx"].cuda(), topk=topk,
                             pool_blocks=pool_blocks, cand_block=cb)
    torch.cuda.synchronize()
    tk, pool = tk.cpu().numpy(), pool.cpu().numpy()
    stats = []
    for b in range(case.B):
        n_vis = case.n_vis[b]
        keys = oc.index_keys(b, np.arange(n_vis))
        s = index_scores(bits(L["q_idx"][b]), bits(L["w_idx"][b]), keys)
        stats.append(check_topk_set(tk[b], np.arange(n_vis), s, topk)["diff"])
        _check_pool(pool[b], s, n_vis, cb, pool_blocks)
    print("near-tie differences per sequence:", stats)


def test_index_full_without_pool_and_repeatable(fk):
    cfg = small_decode(2, B=3, ctx=(40000, 1000, 77778), pages="random", append=0)
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    L = case.layer(0)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    outs = [fk.index_full(gc, ctx_len, max(case.ctx_len), L["q_idx"].cuda(), L["w_idx"].cuda(),
                          topk=512)[0].cpu() for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    for b in range(case.B):
        n_vis = case.n_vis[b]
        s = index_scores(bits(L["q_idx"][b]), bits(L["w_idx"][b]), oc.index_keys(b, np.arange(n_vis)))
        check_topk_set(outs[0][b].numpy(), np.arange(n_vis), s, 512)


@pytest.mark.parametrize("split", [True, False], ids=["split", "one-pass"])
@pytest.mark.parametrize("ctx,pool_blocks,cb,topk", [((65536, 9000, 300), 512, 8, 512),
                                                     ((20000,), 100, 4, 64), ((778,), 200, 8, 512),
                                                     ((60000,), 1024, 16, 300),
                                                     ((50000,), 700, 8, 512)])   # 5,600 slots
def test_reindex_matches_oracle_on_oracle_pool(fk, ctx, pool_blocks, cb, topk, split):
    cfg = small_decode(1, B=len(ctx), ctx=ctx, pages="random", heavy_frac=0.05, append=0)
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    L0, L1 = case.layer(0), case.layer(1)
    pools = np.full((case.B, pool_blocks), -1, np.int32)
    for b in range(case.B):
        _, blocks, _ = full_layer(oc, b, case.n_vis[b], bits(L0["q_idx"][b]), bits(L0["w_idx"][b]), topk,
                                  pool_blocks, cb)
        pools[b, :len(blocks)] = blocks
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    tk = fk.reindex(gc, ctx_len, L1["q_idx"].cuda(), L1["w_idx"].cuda(), torch.from_numpy(pools).cuda(),
                    topk=topk, cand_block=cb, split=split)
    torch.cuda.synchronize()
    tk = tk.cpu().numpy()
    for b in range(case.B):
        pos = pool_positions(pools[b][pools[b] >= 0], case.n_vis[b], cb)
        s = index_scores(bits(L1["q_idx"][b]), bits(L1["w_idx"][b]), oc.index_keys(b, pos))
        check_topk_set(tk[b], pos, s, topk)


def _tied_caches(fk, ctx, factor_of, seed):
    """Caches whose indexer keys are entry 0's key of each sequence times factor_of(n)[j]
    (powers of two): the FP4 codes are equal and the scales shift, so every score is
    exactly factor x the base score on both sides, and the selections are fully
    decided by the lower-index rule among equal scores."""
    from oracle import OracleCache
    cfg = small_decode(1, B=len(ctx), ctx=ctx, H=16, pages="random", heavy_frac=0.0, append=0, seed=seed)
    case = make_decode_case(cfg, "cpu")
    gc = fk.PagedCache.allocate(case.n_pages, case.block_table, device="cuda", ratio=2)
    oc = OracleCache(case.n_pages, case.block_table.numpy(), ratio=2)
    for b in range(case.B):
        x, w, k = case.seq_tokens(b)
        f = torch.as_tensor(factor_of(k.shape[0]), dtype=torch.float32)[:, None]
        k = (k[:1].float() * f).to(torch.bfloat16)
        fk.write_kv(gc.rows(b, b + 1), torch.zeros(1, dtype=torch.int32, device="cuda"), x.cuda()[None].contiguous(),
                    w.cuda()[None].contiguous(), k.cuda()[None].contiguous())
        oc.write(b, 0, None, None, bits(k), latent=False)
    torch.cuda.synchronize()
    return case, gc, oc


@pytest.mark.parametrize("kind", ["all_equal", "three_values"])
def test_tied_scores_resolve_to_lowest_entries(fk, kind):
    # Full top-K, HSI pool and Reindex must equal the oracle exactly: with scores tied
    # in large groups, lower entry indices (and lower block indices) win.
    ctx = (40000, 6000, 900, 2)
    rng = np.random.default_rng(5)
    if kind == "all_equal":
        factor_of = lambda n: np.ones(n)
    else:
        factor_of = lambda n: rng.choice([1.0, 2.0, 4.0], size=n)
    case, gc, oc = _tied_caches(fk, ctx, factor_of, seed=1207 if kind == "all_equal" else 1208)
    L0, L1 = case.layer(0), case.layer(1)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    topk, P, cb = 512, 300, 8
    tk, pool = fk.index_full(gc, ctx_len, max(case.ctx_len), L0["q_idx"].cuda(), L0["w_idx"].cuda(), topk=topk,
                             pool_blocks=P, cand_block=cb)
    tk2 = fk.reindex(gc, ctx_len, L1["q_idx"].cuda(), L1["w_idx"].cuda(), pool, topk=topk, cand_block=cb)
    torch.cuda.synchronize()
    tk, pool, tk2 = tk.cpu().numpy(), pool.cpu().numpy(), tk2.cpu().numpy()
    for b in range(case.B):
        n_vis = case.n_vis[b]
        t, p, _ = full_layer(oc, b, n_vis, bits(L0["q_idx"][b]), bits(L0["w_idx"][b]), topk, P, cb)
        assert np.array_equal(tk[b][tk[b] >= 0], t), f"seq {b}: top-K"
        assert np.array_equal(pool[b][pool[b] >= 0], np.sort(p)), f"seq {b}: pool"
        t2, _ = reindex_layer(oc, b, n_vis, bits(L1["q_idx"][b]), bits(L1["w_idx"][b]), np.sort(p), cb, topk)
        assert np.array_equal(tk2[b][tk2[b] >= 0], t2), f"seq {b}: Reindex"
        if kind == "all_equal" and n_vis > topk:
            assert np.array_equal(t, np.arange(topk))


def _lowest_index_rule(sel, zero, amb, what):
    """sel: selected ids; zero: ids tied at score 0 (the top); amb: ids whose sign of some
    head dot is within rounding of 0, so either side may count them as tied or not.
    Selected ids outside amb must be tied, and no unselected tie below the largest
    selected id may be skipped (the lower index wins among equal scores)."""
    sel = set(int(x) for x in sel)
    assert not (sel - amb) - zero, f"{what}: an id below the tied top was selected"
    top = max(sel)
    skipped = [j for j in zero - amb if j < top and j not in sel]
    assert not skipped, f"{what}: tied ids skipped for higher ones: {skipped[:5]}"


def test_all_negative_head_weights_tie_at_zero(fk):
    # All four indexer head weights negative: every score is <= 0, and the entries whose
    # four head dots are all <= 0 (1 in 16) score exactly -0, the largest value.  Those
    # ties fill the top-K and the pool; the lowest entries and blocks must win, in Full,
    # in the HSI pool and in Reindex (tied pool entries under the second layer's weights).
    ctx = (40000, 65536, 3000)
    cfg = small_decode(1, B=len(ctx), ctx=ctx, pages="random", heavy_frac=0.05, append=0, seed=1209)
    case = make_decode_case(cfg, "cpu")
    oc = oracle_cache_for(case)
    gc = gpu_cache_for(case)
    L0, L1 = case.layer(0), case.layer(1)
    w0, w1 = -L0["w_idx"].abs(), -L1["w_idx"].abs()
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    topk, P, cb = 512, 300, 8
    tk, pool = fk.index_full(gc, ctx_len, max(case.ctx_len), L0["q_idx"].cuda(), w0.cuda(), topk=topk,
                             pool_blocks=P, cand_block=cb)
    tk2 = fk.reindex(gc, ctx_len, L1["q_idx"].cuda(), w1.cuda(), pool, topk=topk, cand_block=cb)
    torch.cuda.synchronize()
    tk, pool, tk2 = tk.cpu().numpy(), pool.cpu().numpy(), tk2.cpu().numpy()

    def ties(q, w, keys):
        s = index_scores(bits(q), bits(w), keys)
        dots = keys @ q.double().numpy().T                       # [n, 4] exact head dots
        amb = (np.abs(dots).min(axis=1) < 1e-5) | ((s < 0) & (s > -1e-5))
        return s, s == 0, amb

    n_tied_top = []
    for b in range(case.B):
        n_vis = case.n_vis[b]
        keys = oc.index_keys(b, np.arange(n_vis))
        s, z, amb = ties(L0["q_idx"][b], w0[b], keys)
        assert s.max() <= 0
        check_topk_set(tk[b], np.arange(n_vis), s, topk)
        sel = tk[b][tk[b] >= 0]
        if z.sum() >= topk:
            n_tied_top.append(b)
            _lowest_index_rule(sel, set(np.flatnonzero(z).tolist()), set(np.flatnonzero(amb).tolist()),
                               f"seq {b} top-K")
        # pool: the newest block last, older blocks by block maximum, lowest block first among ties
        _check_pool(pool[b], s, n_vis, cb, P)
        pv = pool[b][pool[b] >= 0]
        nb = (n_vis + cb - 1) // cb
        assert pv[-1] == nb - 1
        pad = (-n_vis) % cb
        zb = np.concatenate([z, np.zeros(pad, bool)]).reshape(-1, cb).any(axis=1)[:nb - 1]
        ab = np.concatenate([amb, np.zeros(pad, bool)]).reshape(-1, cb).any(axis=1)[:nb - 1]
        if len(pv) > 1 and zb.sum() >= len(pv) - 1:
            _lowest_index_rule(pv[:-1], set(np.flatnonzero(zb).tolist()), set(np.flatnonzero(ab).tolist()),
                               f"seq {b} pool")
        # Reindex over the GPU's pool with the second layer's (negative) weights
        pos = pool_positions(pv, n_vis, cb)
        s2, z2, amb2 = ties(L1["q_idx"][b], w1[b], oc.index_keys(b, pos))
        check_topk_set(tk2[b], pos, s2, topk)
        if z2.sum() >= topk:
            _lowest_index_rule(tk2[b][tk2[b] >= 0], set(pos[z2].tolist()), set(pos[amb2].tolist()),
                               f"seq {b} Reindex")
    assert n_tied_top, "no sequence had K entries tied at the top"
