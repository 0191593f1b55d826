"""HISA-style block-mean pool: block summaries of the indexer keys and the two-stage
selection that scores them.  Test infrastructure.

[P1] §2.3.4 describes HISA (prior work the HSI builds on): the visible prefix is
cut into consecutive blocks; each block keeps the mean of its indexer keys (during
decoding the current block's sum and count are maintained, a new position updates
one block only, finished blocks keep their summary); the first stage scores the
block means with the same indexer query and keeps the best blocks, expanded to
their positions; the second stage scores those positions exactly and keeps the
final top-K.  Readings where the page is silent:
  - a block covers cand_block consecutive entries; its summary is the mean of the
    dequantised keys of its visible entries whose pages are present, summed in
    float32 in entry order and divided once by the count (float32, nearest);
    a block with no such entry has the zero key;
  - the summary is stored like an indexer key (MXFP4: 34 bytes per block), so the
    first stage streams 1/cand_block of the key bytes;
  - no block is forced into the pool (that is HSI's boundary rule, not HISA's);
  - ties in block scores or entry scores go to the lower index.
"""
from __future__ import annotations

import numpy as np

from .fp4 import dequantise_blocks, quantise_blocks
from .indexer import index_scores, reindex_layer


def block_summaries(cache, b: int, n_vis: int, cand_block: int):
    """MXFP4 (codes [nb, 64], scales [nb, 2]) of the block means of sequence b's keys."""
    nb = -(-n_vis // cand_block)
    if nb == 0:
        return np.zeros((0, 64), np.uint8), np.zeros((0, 2), np.uint8)
    js = np.arange(nb * cand_block)
    present = js < n_vis
    pages = cache.block_table[b, np.minimum(js, max(n_vis - 1, 0)) // 64]
    present &= (pages >= 0) & (pages < cache.n_pages)
    keys = np.zeros((nb * cand_block, 64), np.float32)
    if present.any():
        keys[present] = cache.index_keys(b, js[present]).astype(np.float32)   # exact: e2m1 x 2^k
    keys = keys.reshape(nb, cand_block, 64)
    s = np.zeros((nb, 64), np.float32)
    for i in range(cand_block):                      # float32 sum in entry order
        s = (s + keys[:, i, :]).astype(np.float32)
    cnt = present.reshape(nb, cand_block).sum(axis=1).astype(np.float32)
    mean = np.where(cnt[:, None] > 0, s / np.maximum(cnt, 1)[:, None], 0.0).astype(np.float32)
    return quantise_blocks(mean.astype(np.float64))


def hisa_layer(cache, b: int, n_vis: int, q_idx_bits, w_idx_bits, cand_block: int, pool_blocks: int, topk: int):
    """(top-K entries, pool blocks ascending, block scores) of the two-stage selection."""
    codes, scales = block_summaries(cache, b, n_vis, cand_block)
    nb = codes.shape[0]
    if nb == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0)
    mu = dequantise_blocks(codes, scales)
    S = index_scores(q_idx_bits, w_idx_bits, mu)
    order = np.lexsort((np.arange(nb), -S))
    blocks = np.sort(order[:min(pool_blocks, nb)])
    t, _ = reindex_layer(cache, b, n_vis, q_idx_bits, w_idx_bits, blocks, cand_block, topk)
    return t, blocks, S
