"""Pins of the oracle's indexer scores, top-K, HSI pool, Reindex (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import f64_to_bf16_bits, hsi_pool, index_scores, topk_select
from oracle.indexer import pool_positions, reindex_layer, full_layer
from oracle.cache import OracleCache

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def bits(x):
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_scores_closed_form_with_unit_queries():
    # keys k_j = (j - 5) * e_0 + (j % 3) * e_1 ; head h queries a single coordinate
    n = 12
    keys = np.zeros((n, 64))
    keys[:, 0] = np.arange(n) - 5
    keys[:, 1] = np.arange(n) % 3
    q = np.zeros((4, 64))
    q[0, 0] = 1.0          # head 0 sees j - 5 (negative for j < 5 -> ReLU 0)
    q[1, 1] = 2.0          # head 1 sees 2 * (j % 3)
    q[2, 0] = -1.0         # head 2 sees 5 - j
    q[3, 2] = 1.0          # head 3 sees 0
    w = np.array([1.0, 0.5, 4.0, 100.0])
    s = index_scores(bits(q), bits(w), keys)
    j = np.arange(n)
    want = np.maximum(j - 5, 0) * 1.0 + 2 * (j % 3) * 0.5 + np.maximum(5 - j, 0) * 4.0
    assert np.array_equal(s, want)


def test_scores_single_head_positive_dots_is_matrix_vector_product():
    rng = np.random.default_rng(0)
    keys = np.abs(rng.integers(1, 8, size=(50, 64))).astype(np.float64)
    q = np.zeros((4, 64))
    q[0] = np.abs(rng.integers(1, 4, size=64))
    w = np.array([1.0, 0.0, 0.0, 0.0])
    s = index_scores(bits(q), bits(w), keys)
    mv = [sum(int(keys[j, d]) * int(q[0, d]) for d in range(64)) for j in range(50)]
    assert s.tolist() == mv


def _brute_topk(s, k):
    n = len(s)
    chosen = []
    for j in range(n):
        rank = sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j))
        if rank < k:
            chosen.append(j)
    return chosen


@pytest.mark.parametrize("n,k", [(1, 4), (7, 3), (40, 12), (64, 64), (64, 100), (33, 0)])
def test_topk_matches_pairwise_rank_with_ties(n, k):
    rng = np.random.default_rng(n * 7 + k)
    s = rng.integers(-3, 4, size=n).astype(np.float64)       # many ties
    assert topk_select(s, k).tolist() == _brute_topk(s, k)


def _brute_pool(s, width, bs, nb):
    n_blocks = (width + bs - 1) // bs
    bmax = []
    for b in range(n_blocks):
        vals = [s[j] for j in range(b * bs, min(width, (b + 1) * bs))]
        bmax.append(max(vals))
    bmax[(width - 1) // bs] = float("inf")
    chosen = _brute_topk(bmax, nb)
    bitmap = [((j // bs) in chosen) for j in range(width)]
    return chosen, bitmap


@pytest.mark.parametrize("width,bs,nb", [(1, 8, 4), (8, 8, 1), (61, 8, 3), (64, 8, 2), (100, 4, 7),
                                         (100, 8, 100), (77, 1, 10)])
def test_hsi_pool_matches_brute_force(width, bs, nb):
    rng = np.random.default_rng(width + nb)
    s = rng.integers(-5, 6, size=width).astype(np.float64)
    chosen, bitmap = hsi_pool(s, width, bs, nb)
    c2, b2 = _brute_pool(s, width, bs, nb)
    assert chosen.tolist() == c2
    assert bitmap.tolist() == b2
    assert (width - 1) // bs in chosen.tolist()             # newest block always kept


def test_hsi_pool_size_matches_pages_example():
    ex = GOLDEN["hsi_example"]
    rng = np.random.default_rng(5)
    width = 50000
    s = rng.standard_normal(width)
    chosen, bitmap = hsi_pool(s, width, ex["block_size"], ex["blocks"])
    assert len(chosen) == ex["blocks"]
    assert bitmap.sum() == ex["positions"] == ex["blocks"] * ex["block_size"]


def test_pool_contains_topk_when_quota_exceeds_k():
    rng = np.random.default_rng(6)
    for trial in range(20):
        width = int(rng.integers(600, 5000))
        s = rng.standard_normal(width)
        k = 64
        t = topk_select(s, k)
        chosen, bitmap = hsi_pool(s, width, 8, k + 1)
        assert bitmap[t].all()


def _cache_with_keys(keys):
    n = keys.shape[0]
    pages = (n + 63) // 64
    cache = OracleCache(pages, np.arange(pages)[None, :])
    T = 2 * n
    x = np.zeros((T, 512), np.uint16)
    w = np.zeros((T, 512), np.uint16)
    cache.write(0, 0, x, w, bits(keys))
    return cache


def test_reindex_with_full_query_reproduces_full_topk():
    rng = np.random.default_rng(7)
    n = 3000
    keys = rng.standard_normal((n, 64))
    cache = _cache_with_keys(keys)
    q, w = bits(rng.standard_normal((4, 64))), bits(rng.standard_normal(4))
    t, pool, _ = full_layer(cache, 0, n, q, w, 100, pool_blocks=101, cand_block=8)
    t2, _ = reindex_layer(cache, 0, n, q, w, pool, 8, 100)
    assert np.array_equal(t, t2)


def test_pages_reuse_figure_24_positions_pool_10_read_4():
    fig = GOLDEN["p3_reuse_figure"]
    n, want = fig["positions"], fig["read"]
    # one-hot keys: entry j has key e_{j % 64} scaled so distinct queries can rank them
    keys = np.zeros((n, 64))
    keys[np.arange(n), np.arange(n)] = 1.0
    cache = _cache_with_keys(keys)
    pool_members = [2, 4, 7, 10, 11, 15, 17, 19, 20, 23]      # 23 is the newest position
    q_full = np.zeros((4, 64))
    q_full[0, pool_members] = 2.0
    q_full[0, [0, 1, 3]] = 1.0
    w = bits([1.0, 0.0, 0.0, 0.0])
    t_full, pool, s_full = full_layer(cache, 0, n, bits(q_full), w, 4, pool_blocks=fig["pool"],
                                      cand_block=1)
    assert pool_positions(pool, n, 1).tolist() == pool_members
    assert len(pool) == fig["pool"]
    # Reindex query: prefers 0 and 1 (outside the pool) most, then the 4 figure positions
    q_re = np.zeros((4, 64))
    q_re[0, [0, 1]] = 8.0
    q_re[0, want] = 4.0
    q_re[0, [4, 7]] = 1.0
    t_re, _ = reindex_layer(cache, 0, n, bits(q_re), w, pool, 1, 4)
    assert t_re.tolist() == want
