"""Indexer scores, top-K, HSI candidate pool, Full and Reindex layers.  Test infrastructure.

[P1] §2.3.1: a light indexer scores the main-KV entries with an indexer query
and indexer key and keeps the top-K entries per query.  [P1] §2.3.2: a Full
layer scores everything visible and gives a new top-K; a Reindex layer keeps
the shared keys, brings its own indexer query, re-scores and gives its own
top-K; a Reuse layer takes the latest top-K unchanged.  [P1] §2.3.4 (HSI):
the Full layer's scores are max-reduced over blocks of candidate_block_size
positions (the last block padded with -inf), the block holding the newest
visible position is forced in, the best candidate_topk_blocks blocks form the
candidate pool, and Reindex layers score only inside that pool.

Readings where the pages are silent: score s_j = sum_h w_h * max(0, q_h . k_j)
over 4 indexer heads with one 64-d key per entry shared by all heads; the
forced block's value is +inf; ties in scores or block maxima go to the lower
index; fewer candidates than the quota means all are taken.
"""
from __future__ import annotations

import numpy as np

from .fp4 import bf16_bits_to_f64


def index_scores(q_idx_bits, w_idx_bits, keys) -> np.ndarray:
    """s_j = sum_h w_h * ReLU(q_h . k_j) for keys [n, 64]; q_idx [4, 64], w_idx [4] as bf16 bits."""
    q = bf16_bits_to_f64(q_idx_bits)
    w = bf16_bits_to_f64(w_idx_bits)
    keys = np.asarray(keys, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(0, np.float64)
    dots = keys @ q.T                                   # [n, heads]
    return (np.maximum(dots, 0.0) * w[None, :]).sum(axis=1)


def topk_select(scores, k: int, ids=None) -> np.ndarray:
    """The min(k, n) best entries by (score descending, index ascending), returned sorted by index."""
    s = np.asarray(scores, dtype=np.float64)
    ids = np.arange(s.shape[0]) if ids is None else np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -s))                       # primary: -score, secondary: index
    return np.sort(ids[order[:min(k, s.shape[0])]])


def hsi_pool(scores, width: int, block_size: int, topk_blocks: int):
    """Candidate pool from Full-layer scores ([P1] §2.3.4).

    Returns (chosen block ids ascending, boolean bitmap of length width).
    """
    s = np.asarray(scores, dtype=np.float64)[:width]
    if width == 0 or topk_blocks <= 0:
        return np.zeros(0, np.int64), np.zeros(width, bool)
    pad = (-width) % block_size                          # pad the last block with -inf
    padded = np.concatenate([s, np.full(pad, -np.inf)])
    block_max = padded.reshape(-1, block_size).max(axis=-1)
    block_max[(width - 1) // block_size] = np.inf        # newest visible position's block is kept
    n_blocks = block_max.shape[0]
    order = np.lexsort((np.arange(n_blocks), -block_max))
    chosen = np.sort(order[:min(topk_blocks, n_blocks)])
    flags = np.zeros(n_blocks, bool)
    flags[chosen] = True
    bitmap = np.repeat(flags, block_size)[:width]       # expand block flags to positions
    return chosen, bitmap


def full_layer(cache, b: int, n_vis: int, q_idx_bits, w_idx_bits, topk: int,
               pool_blocks: int = 0, cand_block: int = 8):
    """Full mode: score all n_vis visible entries, top-K, optional HSI pool.

    Returns (topk ids ascending, pool block ids ascending, scores).
    """
    keys = cache.index_keys(b, np.arange(n_vis))
    s = index_scores(q_idx_bits, w_idx_bits, keys)
    t = topk_select(s, topk)
    if pool_blocks > 0:
        blocks, _ = hsi_pool(s, n_vis, cand_block, pool_blocks)
    else:
        blocks = np.zeros(0, np.int64)
    return t, blocks, s


def pool_positions(blocks, n_vis: int, cand_block: int) -> np.ndarray:
    """Visible positions covered by the chosen candidate blocks."""
    blocks = np.asarray(blocks, dtype=np.int64)
    if blocks.size == 0:
        return np.zeros(0, np.int64)
    pos = (blocks[:, None] * cand_block + np.arange(cand_block)[None, :]).reshape(-1)
    return pos[pos < n_vis]


def reindex_layer(cache, b: int, n_vis: int, q_idx_bits, w_idx_bits, pool_blocks_ids,
                  cand_block: int, topk: int):
    """Reindex mode: re-score only the pool's positions with this layer's indexer query."""
    pos = pool_positions(pool_blocks_ids, n_vis, cand_block)
    keys = cache.index_keys(b, pos)
    s = index_scores(q_idx_bits, w_idx_bits, keys)
    return topk_select(s, topk, ids=pos), s
