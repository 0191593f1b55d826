"""csa2_index_full_noalloc against csa2_index_full: same kernels, the library's fixed
per-GPU array as workspace instead of the caller's.  Two calls in a row on one stream,
the second on a smaller input, so that the array still holds the first call's
contents; both must equal the allocating entry point bit for bit (top-K and pool are
integer results)."""
import pytest
import torch

from synth import make_decode_case, small_decode
from tests.helpers import gpu_cache_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    return m


# (ctx per sequence, topk, pool_blocks, cand_block); the second is smaller in every way
CALLS = [
    ((65536, 3000, 0, 40002, 2, 65534, 9000, 131070), 512, 512, 8),
    ((20000, 14), 64, 40, 4),
]


def _run(fk, ctx, topk, pool_blocks, cb, seed):
    cfg = small_decode(1, B=len(ctx), ctx=ctx, seed=seed, pages="random", heavy_frac=0.05, append=0,
                       layers=small_decode(1, B=1, ctx=(2,)).layers)
    case = make_decode_case(cfg, "cpu")
    gc = gpu_cache_for(case)
    L = case.layer(0)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    max_ctx = max(case.ctx_len)
    q, w = L["q_idx"].cuda(), L["w_idx"].cuda()
    # the allocating entry point, its workspace filled with garbage first
    ws = fk.workspace(fk.FN_INDEX_FULL, device="cuda", B=len(ctx), max_ctx=max_ctx, topk=topk,
                      pool_blocks=pool_blocks, ratio=gc.ratio)
    if ws is not None:
        ws.fill_(0xA5)
    want_tk, want_pool = fk.index_full(gc, ctx_len, max_ctx, q, w, topk=topk, pool_blocks=pool_blocks,
                                       cand_block=cb, ws=ws)
    tk = torch.full((len(ctx), topk), -7, dtype=torch.int32, device="cuda")
    pool = torch.full((len(ctx), pool_blocks), -7, dtype=torch.int32, device="cuda")
    fk.index_full_noalloc(gc, ctx_len, max_ctx, q, w, tk, pool, topk=topk, pool_blocks=pool_blocks,
                          cand_block=cb)
    torch.cuda.synchronize()
    return (want_tk.cpu(), want_pool.cpu()), (tk.cpu(), pool.cpu())


def test_noalloc_matches_allocating_entry_on_two_calls(fk):
    for i, (ctx, topk, pool_blocks, cb) in enumerate(CALLS):
        print(f"call {i}: B={len(ctx)} max_ctx={max(ctx)} topk={topk} pool={pool_blocks} cb={cb}", flush=True)
        (want_tk, want_pool), (tk, pool) = _run(fk, ctx, topk, pool_blocks, cb, seed=11 + i)
        assert torch.equal(tk, want_tk), f"call {i}: top-K differs"
        assert torch.equal(pool, want_pool), f"call {i}: pool differs"
        assert (tk >= 0).any() and (pool >= 0).any()

