"""GPU tests of the layer-schedule runner (csa2_schedule_*).

The captured graph must give, bit for bit, what the same calls give one by one
(it runs the same kernels on the same buffers), on every replay.  Against the
oracle's run_decode, for every layer of every sequence checked: Full selections
and pools up to near-ties, Reindex selections over the GPU's own pool, Reuse
keeping the previous selection, and attention on the GPU's own selection within
the 2e-3 bar (lse within 1e-4).
Schedules from [P1] §2.3.3: the decoder's [Full + 3 Reuse] + 4 x [Reindex + 3 Reuse]
(ratio 1, pool 2048 x 8) and the encoder's [Full + 5 Reuse] x 3 (ratio 2).
"""
import numpy as np
import pytest
import torch

from oracle.indexer import index_scores, pool_positions
from oracle.schedule import run_decode
from synth import make_decode_case, small_decode
from synth.configs import DECODER_SCHEDULE as DECODER, ENCODER_SCHEDULE as ENCODER
from tests.helpers import (AttentionReport, bits, check_pool_set, check_topk_set, gpu_cache_for,
                           oracle_cache_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fk():
    import fp4_kv_cache_write_amd as m
    m.lib()
    return m


def _layers(case, H):
    ls = []
    for l, sp in enumerate(case.cfg.layers):
        L = case.layer(l)
        ls.append(dict(mode=sp.mode, pool_blocks=sp.pool_blocks, q=L["q"].cuda(), q_idx=L["q_idx"].cuda(),
                       w_idx=L["w_idx"].cuda(), swa=L["swa"].cuda(),
                       out=torch.empty((case.B, H, 512), dtype=torch.bfloat16, device="cuda"),
                       lse=torch.empty((case.B, H), dtype=torch.float32, device="cuda")))
    return ls


def _eager(fk, gc, case, ctx_len, layers, write):
    """The same calls one by one; returns per layer (out, lse, selection)."""
    if write is not None:
        fk.write_kv(gc, write["start"], write["x"], write["w"], write["k"])
    res, sel, pool, pb = [], None, None, 0
    for L in layers:
        if L["mode"] == "full":
            pb = L["pool_blocks"]
            sel, p = fk.index_full(gc, ctx_len, max(case.ctx_len), L["q_idx"], L["w_idx"], topk=512,
                                   pool_blocks=pb, cand_block=8)
            if pb > 0:
                pool = p
        elif L["mode"] == "reindex":
            sel = fk.reindex(gc, ctx_len, L["q_idx"], L["w_idx"], pool, topk=512, cand_block=8)
        o, lse = fk.sparse_decode(gc, ctx_len, L["q"], sel, L["swa"])
        res.append((o.clone(), lse.clone(), sel.clone(), None if pool is None else pool.clone()))
    torch.cuda.synchronize()
    return res


def _run(fk, cfg_layers, ratio, ctx, write_last):
    cfg = small_decode(5 if ratio == 1 else 1, B=len(ctx), ctx=ctx, H=16, pages="random", heavy_frac=0.05,
                       append=0, layers=cfg_layers, ratio=ratio)
    case = make_decode_case(cfg, "cpu")
    gc = gpu_cache_for(case)
    ctx_len = torch.tensor(case.ctx_len, dtype=torch.int32, device="cuda")
    write = None
    if write_last:   # the step re-writes each sequence's newest entry (bit-identical bytes)
        xs, ws_, ks = [], [], []
        for b in range(case.B):
            x, w, k = case.seq_tokens(b)
            xs.append(x[-ratio:])
            ws_.append(None if w is None else w[-ratio:])
            ks.append(k[-1:])
        write = dict(x=torch.stack(xs).cuda(), w=None if ratio == 1 else torch.stack(ws_).cuda(),
                     k=torch.stack(ks).cuda(),
                     start=torch.tensor([L - ratio for L in case.ctx_len], dtype=torch.int32, device="cuda"))
    layers = _layers(case, 16)
    sch = fk.Schedule(gc, ctx_len, max(case.ctx_len), layers, W=cfg.window, write=write)
    outs = []
    for _ in range(3):   # each replay checked; eager fills and a sync between replays
        for L in layers:
            L["out"].zero_()
            L["lse"].zero_()
        sch.launch()
        torch.cuda.synchronize()
        outs.append([(L["out"].clone(), L["lse"].clone()) for L in layers])
    sch.close()
    eager = _eager(fk, gc, case, ctx_len, layers, write)
    for l in range(len(layers)):
        for rep in outs:
            assert torch.equal(rep[l][0], eager[l][0]), f"layer {l}: out differs from the calls"
            assert torch.equal(rep[l][1], eager[l][1]), f"layer {l}: lse differs from the calls"
    return case, layers, eager


def _check_oracle(case, layers, eager, seqs, cand_block=8, topk=512):
    """Every layer of every sequence in seqs against the oracle (module docstring)."""
    oc = oracle_cache_for(case, seqs=seqs)
    specs = [dict(mode=L["mode"], pool_blocks=L["pool_blocks"], q=bits(L["q"].cpu()), q_idx=bits(L["q_idx"].cpu()),
                  w_idx=bits(L["w_idx"].cpu()), swa=bits(L["swa"].cpu())) for L in layers]
    sels = [e[2].cpu().numpy() for e in eager]
    attend = [{b: sels[l][b][sels[l][b] >= 0] for b in seqs} for l in range(len(layers))]
    ref = run_decode(oc, case.ctx_len, specs, topk=topk, W=case.cfg.window, cand_block=cand_block, seqs=seqs,
                     attend_on=attend)
    rep, same = AttentionReport(), 0
    for b in seqs:
        nv = case.n_vis[b]
        g_pool = None
        for l, (o, lse, sel, pool) in enumerate(eager):
            g = sels[l][b]
            sp = specs[l]
            if sp["mode"] == "full":
                s = index_scores(sp["q_idx"][b], sp["w_idx"][b], oc.index_keys(b, np.arange(nv)))
                check_topk_set(g, np.arange(nv), s, topk)
                if sp["pool_blocks"] > 0:
                    p = pool[b].cpu().numpy()
                    check_pool_set(p, s, nv, cand_block, sp["pool_blocks"])
                    g_pool = p[p >= 0]
            elif sp["mode"] == "reindex":
                pos = pool_positions(g_pool, nv, cand_block)
                s2 = index_scores(sp["q_idx"][b], sp["w_idx"][b], oc.index_keys(b, pos))
                check_topk_set(g, pos, s2, topk)
            else:
                assert np.array_equal(g, sels[l - 1][b]), f"layer {l}: Reuse changed the selection"
            rep.check(bits(o[b].cpu()), ref[l]["o"][b], lse[b].cpu().numpy(), ref[l]["lse"][b])
            same += int(np.array_equal(g[g >= 0], ref[l]["topk"][b]))
    assert rep.n == len(seqs) * len(eager)
    return rep, same


def test_decoder_schedule_equals_calls_and_oracle(fk):
    case, layers, eager = _run(fk, DECODER, 1, (9000, 20000), write_last=True)
    rep, same = _check_oracle(case, layers, eager, seqs=(0, 1))
    print(f"decoder schedule: {rep}; {same}/{rep.n} selections identical to the oracle's")


def test_encoder_schedule_equals_calls_and_oracle(fk):
    case, layers, eager = _run(fk, ENCODER, 2, (4000, 12000), write_last=True)
    rep, same = _check_oracle(case, layers, eager, seqs=(0, 1))
    print(f"encoder schedule: {rep}; {same}/{rep.n} selections identical to the oracle's")
