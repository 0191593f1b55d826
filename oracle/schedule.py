"""Layer schedules and chunked prefill, end to end.  Test infrastructure.

[P1] §2.3.2: Full, Reindex and Reuse layers share one cache; each layer
computes its own main query and window.  [P1] §2.3.3: an encoder block is one
Full layer then Reuse layers; the decoder's later blocks start with a Reindex
layer that searches the Full layer's candidate pool.  [P3]
("選ぶ位置は同じでも、情報の混ぜ方は変わる"): Reuse keeps the positions while the
query, and so the weights, change.

Visibility ([P3], causal mask): at ratio 2 entry j merges tokens 2j and 2j+1, so
a query at token t sees entries with 2j+1 <= t, i.e. floor((t+1)/2) of them; at
ratio 1 ([P1] §2.3.1, the decoder) entry j is token j and t sees t+1 entries.  A
decode query for a context of L tokens sits at t = L-1.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import gather_rows, sparse_attention
from .indexer import full_layer, index_scores, reindex_layer, topk_select


def n_visible(t: int, ratio: int = 2) -> int:
    return (t + 1) // ratio


def run_decode(cache, ctx_len, layers, topk: int = 512, W: int = 128, cand_block: int = 8,
               sm_scale: float | None = None, seqs=None, attend_on=None):
    """Decode one query per sequence through `layers`.

    layers: list of dicts with mode ("full"|"reindex"|"reuse"), pool_blocks and
    the layer's bf16-bit inputs q [B,H,512], q_idx [B,4,64], w_idx [B,4],
    swa [B,W,512].  Returns per layer a dict with topk[b], pool[b] (block ids),
    o[b] (float64 [H,512]) and lse[b] for every b in seqs.
    attend_on: optional, per layer a dict b -> entry ids.  Where given, that
    layer's attention for b reads those entries instead of the layer's own
    selection (a selection that differs only by near-tied scores is as correct,
    and its attention output is then compared on equal terms); topk[b] and
    pool[b] stay this function's own selections.
    """
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(512.0)
    B = len(ctx_len)
    seqs = range(B) if seqs is None else seqs
    out = []
    cur_t = {b: None for b in seqs}
    cur_pool = {b: np.zeros(0, np.int64) for b in seqs}
    for spec in layers:
        res = {"topk": {}, "pool": {}, "o": {}, "lse": {}}
        for b in seqs:
            t = ctx_len[b] - 1
            nv = n_visible(t, getattr(cache, "ratio", 2))
            if spec["mode"] == "full":
                tk, pool, _ = full_layer(cache, b, nv, spec["q_idx"][b], spec["w_idx"][b], topk,
                                         spec.get("pool_blocks", 0), cand_block)
                cur_t[b] = tk
                if spec.get("pool_blocks", 0) > 0:
                    cur_pool[b] = pool
            elif spec["mode"] == "reindex":
                tk, _ = reindex_layer(cache, b, nv, spec["q_idx"][b], spec["w_idx"][b], cur_pool[b],
                                      cand_block, topk)
                cur_t[b] = tk
            elif spec["mode"] == "reuse":
                assert cur_t[b] is not None, "Reuse needs an earlier Full or Reindex layer"
            else:
                raise ValueError(spec["mode"])
            sel = cur_t[b]
            if attend_on is not None and b in attend_on[len(out)]:
                sel = attend_on[len(out)][b]
            rows = gather_rows(cache, b, sel, spec["swa"][b], t, W)
            o, lse = sparse_attention(spec["q"][b], rows, sm_scale)
            res["topk"][b] = cur_t[b]
            res["pool"][b] = cur_pool[b]
            res["o"][b] = o
            res["lse"][b] = lse
        out.append(res)
    return out


def run_prefill(cache, prior_len, C: int, q, q_idx, w_idx, local, topk: int = 512, W: int = 128,
                sm_scale: float | None = None, queries=None, attend_on=None):
    """Chunked prefill after the chunk's entries were written.

    q [B,C,H,512], q_idx [B,C,4,64], w_idx [B,C,4], local [B,W-1+C,512] (window
    rows for positions prior-W+1 .. prior+C-1) as bf16 bits.  queries: list of
    (b, i) pairs to evaluate (default: all).  Returns dict (b,i) -> (topk, o, lse).
    attend_on: optional dict (b, i) -> entry ids; where given, the query's
    attention reads those entries instead of its own top-K (which is still the
    returned topk), as in run_decode.
    """
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(512.0)
    assert getattr(cache, "ratio", 2) == 2, "chunked prefill is the encoder's (ratio 2) path"
    B = len(prior_len)
    if queries is None:
        queries = [(b, i) for b in range(B) for i in range(C)]
    out = {}
    keys_cache = {}
    for b, i in queries:
        t = prior_len[b] + i
        nv = n_visible(t)
        if b not in keys_cache:
            last = n_visible(prior_len[b] + C - 1)
            keys_cache[b] = cache.index_keys(b, np.arange(last))
        s = index_scores(q_idx[b, i], w_idx[b, i], keys_cache[b][:nv])
        tk = topk_select(s, topk)
        # the window ring for this query: slot pos % W holds local row pos - (prior - W + 1)
        ring = np.zeros((W, local.shape[-1]), dtype=np.uint16)
        for pos in range(max(0, t - W + 1), t + 1):
            ring[pos % W] = local[b, pos - (prior_len[b] - W + 1)]
        sel = tk if attend_on is None or (b, i) not in attend_on else attend_on[(b, i)]
        rows = gather_rows(cache, b, sel, ring, t, W)
        o, lse = sparse_attention(q[b, i], rows, sm_scale)
        out[(b, i)] = (tk, o, lse)
    return out
