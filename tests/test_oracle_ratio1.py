"""Pins of the oracle's ratio-1 cache (one entry per token, the decoder's case) (CPU only).

[P1] §2.3.1: the compressor has a ratio-1 special case that leaves the decoder's
main KV uncompressed, one entry per token, for per-token addressability; the
decoder's Full layer then builds the HSI pool of [P1] §2.3.4 (2048 blocks of 8
positions = 16384 candidates) for its Reindex layers.
"""
import math

import numpy as np

from oracle import OracleCache, bf16_bits_to_f64, f64_to_bf16_bits, quantise_blocks
from oracle.attention import window_positions
from oracle.schedule import n_visible, run_decode


def bits(x):
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def _dense_attention(q, rows, scale):
    """Softmax attention per head with math.exp and math.fsum."""
    out = np.zeros((q.shape[0], rows.shape[1]))
    for h in range(q.shape[0]):
        z = [scale * math.fsum(q[h] * rows[r]) for r in range(rows.shape[0])]
        m = max(z)
        e = [math.exp(v - m) for v in z]
        tot = math.fsum(e)
        for d in range(rows.shape[1]):
            out[h, d] = math.fsum(e[r] * rows[r, d] for r in range(rows.shape[0])) / tot
    return out


def test_ratio1_entry_equals_ratio2_entry_with_unit_weights():
    # At ratio 2, the pair (x_j, y_j) with weights (1, 0) merges to x_j exactly, so its
    # stored entry must equal, byte for byte, the ratio-1 entry of token x_j.
    rng = np.random.default_rng(11)
    n = 150
    bt = np.array([[2, 0, 1]])
    x = bits(rng.standard_normal((n, 512)))
    y = bits(rng.standard_normal((n, 512)))
    k = bits(rng.standard_normal((n, 64)))
    r1 = OracleCache(3, bt, ratio=1)
    r1.write(0, 10, x, None, k)                       # entries 10 .. 159
    x2 = np.empty((2 * n, 512), np.uint16)
    x2[0::2], x2[1::2] = x, y
    w2 = np.zeros((2 * n, 512), np.uint16)
    w2[0::2] = 0x3F80                                 # bf16 1.0; odd tokens weighted 0
    r2 = OracleCache(3, bt, ratio=2)
    r2.write(0, 20, x2, w2, k)                        # entries 10 .. 159
    for name in ("lat_codes", "lat_scales", "idx_codes", "idx_scales"):
        assert np.array_equal(getattr(r1, name), getattr(r2, name)), name
    # entry 10 + i is token i, quantised as it is, in the page the table names
    for i in (0, 53, 54, 149):
        j = 10 + i
        pg, sl = bt[0, j // 64], j % 64
        c, u = quantise_blocks(bf16_bits_to_f64(x[i]))
        assert np.array_equal(r1.lat_codes[pg, sl], (c[0::2] | (c[1::2] << 4)).astype(np.uint8))
        assert np.array_equal(r1.lat_scales[pg, sl], u)
    assert not r1.lat_codes[2, :10].any()             # nothing before entry 10


def test_ratio1_visibility():
    for t in (0, 1, 2, 127, 4095, 65535):
        assert n_visible(t, 1) == t + 1
        assert n_visible(t, 2) == (t + 1) // 2
    assert n_visible(8) == 4                          # ratio 2 stays the default


def test_ratio1_decode_sees_every_token_and_equals_dense():
    # 70 tokens at ratio 1, top-K covering the context: the Full layer selects every
    # entry 0..69 (the newest included) and attention equals dense attention over
    # those entries plus the window.
    rng = np.random.default_rng(12)
    L, W, H = 70, 16, 2
    bt = np.array([[1, 0]])
    cache = OracleCache(2, bt, ratio=1)
    cache.write(0, 0, bits(rng.standard_normal((L, 512))), None, bits(rng.standard_normal((L, 64))))
    q = bits(rng.standard_normal((H, 512)))
    swa = bits(rng.standard_normal((W, 512)))
    layers = [dict(mode="full", pool_blocks=0, q=q[None], q_idx=bits(rng.standard_normal((1, 4, 64))),
                   w_idx=bits(rng.standard_normal((1, 4))), swa=swa[None])]
    res = run_decode(cache, [L], layers, topk=128, W=W)
    assert res[0]["topk"][0].tolist() == list(range(L))
    t = L - 1
    rows = np.concatenate([cache.latent(0, np.arange(L)), bf16_bits_to_f64(swa)[window_positions(t, W) % W]])
    dense = _dense_attention(bf16_bits_to_f64(q), rows, 1 / math.sqrt(512))
    assert np.allclose(res[0]["o"][0], dense, rtol=1e-12, atol=1e-12)


def test_ratio1_pool_of_2048_blocks_bounds_reindex():
    # The pages' HSI setting: 2048 blocks of 8 positions = 16384 candidates.  Over
    # 20000 tokens at ratio 1 (2500 blocks), the pool holds 2048 distinct blocks,
    # among them the newest (forced), and Reindex selects only pooled positions.
    rng = np.random.default_rng(13)
    L = 20000
    pages = (L + 63) // 64
    bt = rng.permutation(pages)[None, :]
    cache = OracleCache(pages, bt, ratio=1)
    cache.write(0, 0, None, None, bits(rng.standard_normal((L, 64))), latent=False)
    q_idx = [bits(rng.standard_normal((1, 4, 64))) for _ in range(2)]
    w_idx = [bits(rng.standard_normal((1, 4))) for _ in range(2)]
    from oracle.indexer import full_layer, reindex_layer
    tk, pool, _ = full_layer(cache, 0, n_visible(L - 1, 1), q_idx[0][0], w_idx[0][0], 512, 2048, 8)
    assert len(pool) == 2048 and len(set(pool.tolist())) == 2048
    assert (L - 1) // 8 in set(pool.tolist())
    tk2, _ = reindex_layer(cache, 0, n_visible(L - 1, 1), q_idx[1][0], w_idx[1][0], pool, 8, 512)
    assert len(tk2) == 512 and set((tk2 // 8).tolist()) <= set(pool.tolist())
