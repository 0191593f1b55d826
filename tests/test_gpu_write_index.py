"""csa2_write_index_full against csa2_write_kv followed by csa2_index_full on the same
stream: the same cache bytes and the same selections (top-K and pool), bit for bit.

The cases put the written entries where the fused scan must store them before it reads
them: the last entry of a chunk, the first of the next, a page's first entry, entry 0,
writes crossing a chunk or a page boundary, written entries past the visible context
(stored, not scored), an odd start at ratio 2 (nothing written), and an absent page
under a written entry; a 70-entry write, which the call runs as two launches, too.
"""
import pytest
import torch

from synth import LayerSpec, make_decode_case, small_decode
from tests.helpers import gpu_cache_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    return m


def _compare(fk, case, start, ctx, absent=None, topk=128, pool_blocks=40, cb=8):
    """Run both paths on clones of one pre-built cache; absent = (b, page slot) to unmap."""
    base = gpu_cache_for(case)
    c1, c2 = base.clone(), base.clone()
    if absent is not None:
        for c in (c1, c2):
            c.block_table[absent[0], absent[1]] = -1
    xa, wa, ka, _ = case.append_tokens()
    x, k = xa.cuda(), ka.cuda()
    w = None if wa is None else wa.cuda()
    start, ctx = start.cuda(), ctx.cuda()
    max_ctx = int(ctx.max())
    L = case.layer(0)
    q_idx, w_idx = L["q_idx"].cuda(), L["w_idx"].cuda()
    fk.write_kv(c1, start, x, w, k)
    tk1, p1 = fk.index_full(c1, ctx, max_ctx, q_idx, w_idx, topk=topk, pool_blocks=pool_blocks, cand_block=cb)
    tk2, p2 = fk.write_index_full(c2, start, x, w, k, ctx, max_ctx, q_idx, w_idx, topk=topk,
                                  pool_blocks=pool_blocks, cand_block=cb)
    torch.cuda.synchronize()
    for name in ("lat_codes", "lat_scales", "idx_codes", "idx_scales"):
        a, b = getattr(c1, name), getattr(c2, name)
        assert torch.equal(a, b), f"{name}: {int((a != b).sum())} bytes differ"
    assert not torch.equal(c1.idx_codes, base.idx_codes), "the write changed nothing"
    assert torch.equal(tk1, tk2), "top-K differs"
    if pool_blocks > 0:
        assert torch.equal(p1, p2), "pool differs"
    return tk1


def test_decode_pair_write_at_chunk_and_page_edges(fk):
    # newest entry: 4095 (last of chunk 0), 4096 (first of chunk 1), 0, 64 (first of
    # page 1), 10000, 9999
    ctx = (8192, 8194, 2, 130, 20002, 20000)
    cfg = small_decode(1, B=len(ctx), ctx=ctx, H=16, pages="random", append=2, topk=128,
                       layers=(LayerSpec("full", 40),))
    case = make_decode_case(cfg, "cpu")
    _, _, _, start = case.append_tokens()
    _compare(fk, case, start, torch.tensor(case.ctx_len, dtype=torch.int32))


def test_decoder_ratio1_single_token_write(fk):
    ctx = (4096, 4097, 1, 65, 9000)
    cfg = small_decode(5, B=len(ctx), ctx=ctx, H=16, pages="random", append=1, topk=128, ratio=1,
                       layers=(LayerSpec("full", 40),))
    case = make_decode_case(cfg, "cpu")
    _, _, _, start = case.append_tokens()
    _compare(fk, case, start, torch.tensor(case.ctx_len, dtype=torch.int32))


def test_two_entry_write_across_edges_with_invisible_odd_and_absent(fk):
    # 2 entries per sequence, the most the scan writes itself.  Seq 0: entries 4095, 4096
    # (one in each chunk); seq 1: 63, 64 (one in each page); seq 2: the context stops
    # after the first (the second is stored, not scored); seq 3: odd start (nothing
    # written); seq 4: its second entry's page is unmapped; seq 5: entries 0, 1.
    A = 4
    ctx = (8190 + A, 126 + A, 2000 + A, 5000 + A, 126 + A, A)
    cfg = small_decode(1, B=len(ctx), ctx=ctx, H=16, pages="random", append=A, topk=128,
                       layers=(LayerSpec("full", 40),))
    case = make_decode_case(cfg, "cpu")
    _, _, _, start = case.append_tokens()
    start = start.clone()
    start[3] += 1
    ctx_t = torch.tensor(case.ctx_len, dtype=torch.int32)
    ctx_t[2] -= 2
    _compare(fk, case, start, ctx_t, absent=(4, 1))


def test_multi_entry_write_runs_as_two_launches(fk):
    # 70 entries per sequence (more than the scan writes itself).  Seq 0: entries 4060..4129 (chunk 0 -> 1, pages 63..64);
    # seq 1: same, but the context stops 40 entries into the write (the rest is stored,
    # not scored); seq 2: odd start (nothing written); seq 3: short sequence whose
    # written page 1 is unmapped; seq 4: a write far from the end of its chunk.
    A = 140
    ctx = (8120 + A, 8120 + A, 3000 + A, 60 + A, 12000 + A)
    cfg = small_decode(1, B=len(ctx), ctx=ctx, H=16, pages="random", append=A, topk=128,
                       layers=(LayerSpec("full", 40),))
    case = make_decode_case(cfg, "cpu")
    _, _, _, start = case.append_tokens()
    start = start.clone()
    start[2] += 1                                  # odd: the write skips sequence 2
    ctx_t = torch.tensor(case.ctx_len, dtype=torch.int32)
    ctx_t[1] = 8120 + 80                           # entries 4100..4129 of seq 1 are past its context
    _compare(fk, case, start, ctx_t, absent=(3, 1))
