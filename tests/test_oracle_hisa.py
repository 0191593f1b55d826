"""Pins of the oracle's HISA block-mean pool (oracle/hisa.py): one-entry blocks
reduce to the Full layer, block means of equal keys are that key, partial blocks
average what they hold, and a hand-computed float32 sum on a tiny case."""
import numpy as np

from oracle import (OracleCache, block_summaries, dequantise_blocks, f64_to_bf16_bits, full_layer, hisa_layer,
                    quantise_blocks)


def _cache(keys_f64, n_pages=None, perm=True, seed=0):
    """Ratio-2 oracle cache holding only indexer keys (one per entry)."""
    n = keys_f64.shape[0]
    n_pages = n_pages or -(-n // 64)
    rng = np.random.default_rng(seed)
    bt = (rng.permutation(n_pages) if perm else np.arange(n_pages))[None].astype(np.int64)
    oc = OracleCache(n_pages, bt)
    oc.write(0, 0, None, None, f64_to_bf16_bits(keys_f64), latent=False)
    return oc


def test_one_entry_blocks_reduce_to_the_full_layer():
    # With blocks of one entry the block key is the entry's key requantised (the value
    # round-trips), so stage 1 ranks entries by their exact scores and stage 2 over a
    # pool of >= K blocks returns the Full layer's top-K.
    rng = np.random.default_rng(1)
    n = 3000
    keys = rng.standard_normal((n, 64)) * np.where(rng.random((n, 1)) < 0.05, 4.0, 1.0)
    oc = _cache(keys)
    q = f64_to_bf16_bits(rng.standard_normal((4, 64)))
    w = f64_to_bf16_bits(rng.standard_normal(4))
    t_full, _, s = full_layer(oc, 0, n, q, w, 200, 0, 1)
    t, blocks, S = hisa_layer(oc, 0, n, q, w, 1, 600, 200)
    assert np.array_equal(S, s)
    assert np.array_equal(t, t_full)
    assert set(t.tolist()) <= set(blocks.tolist())


def test_equal_keys_in_a_block_give_that_key():
    rng = np.random.default_rng(2)
    base = rng.standard_normal((40, 64))
    keys = np.repeat(base, 8, axis=0)              # 40 blocks of 8 equal keys
    oc = _cache(keys)
    codes, scales = block_summaries(oc, 0, 320, 8)
    want = oc.index_keys(0, np.arange(0, 320, 8))
    assert np.array_equal(dequantise_blocks(codes, scales), want)


def test_partial_last_block_and_hand_sum():
    # 37 entries in blocks of 4: the last block holds one entry.  Block means are the
    # float32 sum in entry order divided by the count, then MX-quantised.
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((37, 64)) * np.ldexp(1.0, rng.integers(-6, 7, size=(37, 1)))
    oc = _cache(keys, perm=False)
    codes, scales = block_summaries(oc, 0, 37, 4)
    assert codes.shape == (10, 64)
    k = oc.index_keys(0, np.arange(37)).astype(np.float32)
    for blk in range(10):
        rows = range(4 * blk, min(4 * blk + 4, 37))
        acc = [np.float32(0.0)] * 64
        for j in rows:
            acc = [np.float32(a + k[j, c]) for c, a in enumerate(acc)]
        mean = np.array([np.float32(a / np.float32(len(rows))) for a in acc], np.float64)
        c2, s2 = quantise_blocks(mean[None])
        assert np.array_equal(codes[blk], c2[0]) and np.array_equal(scales[blk], s2[0]), blk
    assert np.array_equal(dequantise_blocks(codes[9:], scales[9:])[0], oc.index_keys(0, [36])[0])


def test_pool_is_the_best_block_means_by_brute_force():
    rng = np.random.default_rng(4)
    n, cb, P = 500, 8, 13
    oc = _cache(rng.standard_normal((n, 64)))
    q = f64_to_bf16_bits(rng.standard_normal((4, 64)))
    w = f64_to_bf16_bits(np.abs(rng.standard_normal(4)))
    t, blocks, S = hisa_layer(oc, 0, n, q, w, cb, P, 40)
    best = sorted(range(len(S)), key=lambda i: (-S[i], i))[:P]
    assert blocks.tolist() == sorted(best)
    pos = [j for blk in blocks for j in range(blk * cb, min(blk * cb + cb, n))]
    from oracle import index_scores
    s = index_scores(q, w, oc.index_keys(0, pos))
    want = sorted(sorted(range(len(pos)), key=lambda i: (-s[i], pos[i]))[:40])
    assert t.tolist() == sorted(pos[i] for i in want)
