"""Pins of the oracle's sparse attention, Reuse, causality and schedules (CPU only)."""
import math

import numpy as np
import pytest

from oracle import OracleCache, bf16_bits_to_f64, f64_to_bf16_bits, sparse_attention
from oracle.attention import gather_rows, window_positions
from oracle.schedule import run_decode, run_prefill, n_visible


def bits(x):
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


def _rand_cache(rng, n_entries, pages_perm=True):
    pages = (n_entries + 63) // 64
    bt = (rng.permutation(pages) if pages_perm else np.arange(pages))[None, :]
    cache = OracleCache(pages, bt)
    T = 2 * n_entries
    x = bits(rng.standard_normal((T, 512)))
    w = bits(rng.uniform(0.1, 1.0, size=(T, 512)))
    k = bits(rng.standard_normal((n_entries, 64)))
    cache.write(0, 0, x, w, k)
    return cache


def _dense_attention_loops(q, rows, scale):
    """Softmax attention written out per head with math.exp and math.fsum."""
    H, R = q.shape[0], rows.shape[0]
    out = np.zeros((H, rows.shape[1]))
    for h in range(H):
        z = [scale * math.fsum(q[h] * rows[r]) for r in range(R)]
        m = max(z)
        e = [math.exp(v - m) for v in z]
        tot = math.fsum(e)
        for d in range(rows.shape[1]):
            out[h, d] = math.fsum(e[r] * rows[r, d] for r in range(R)) / tot
    return out


def test_sparse_equals_dense_when_topk_covers_context():
    rng = np.random.default_rng(0)
    n = 90                                        # 180 tokens, fewer visible entries than K
    cache = _rand_cache(rng, n)
    W, H = 128, 3
    t = 2 * n - 1
    swa = bits(rng.standard_normal((W, 512)))
    q = bits(rng.standard_normal((H, 512)))
    layers = [dict(mode="full", pool_blocks=0, q=q[None], q_idx=bits(rng.standard_normal((1, 4, 64))),
                   w_idx=bits(rng.standard_normal((1, 4))), swa=swa[None])]
    res = run_decode(cache, [2 * n], layers, topk=512, W=W)
    assert res[0]["topk"][0].tolist() == list(range(n))
    # dense: every visible entry, in order, plus the window rows for t-127..t
    rows = np.concatenate([cache.latent(0, np.arange(n)),
                           bf16_bits_to_f64(swa)[window_positions(t, W) % W]])
    dense = _dense_attention_loops(bf16_bits_to_f64(q), rows, 1 / math.sqrt(512))
    assert np.allclose(res[0]["o"][0], dense, rtol=1e-12, atol=1e-12)


def test_softmax_weights_convexity_and_single_row():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((37, 512))
    q = bits(rng.standard_normal((4, 512)))
    o, lse = sparse_attention(q, rows, 0.05)
    assert np.all(o <= rows.max(axis=0) + 1e-12) and np.all(o >= rows.min(axis=0) - 1e-12)
    # constant rows -> output equals that row (weights sum to one)
    r = np.tile(rng.standard_normal((1, 512)), (37, 1))
    o, _ = sparse_attention(q, r, 0.05)
    assert np.allclose(o, r[:4], rtol=0, atol=1e-12)
    o, lse = sparse_attention(q, rows[:1], 0.05)
    assert np.array_equal(o, np.tile(rows[:1], (4, 1)))
    z = 0.05 * bf16_bits_to_f64(q) @ rows[:1].T
    assert np.allclose(lse, z[:, 0], atol=1e-12)


def test_reuse_reads_exactly_the_selected_entries():
    rng = np.random.default_rng(2)
    n = 1500
    cache = _rand_cache(rng, n)
    W, H = 128, 4
    mk = lambda: dict(q=bits(rng.standard_normal((1, H, 512))),
                      q_idx=bits(rng.standard_normal((1, 4, 64))),
                      w_idx=bits(rng.standard_normal((1, 4))), swa=bits(rng.standard_normal((1, W, 512))))
    layers = [dict(mode="full", pool_blocks=80, **mk()), dict(mode="reindex", **mk()),
              dict(mode="reuse", **mk())]
    res = run_decode(cache, [2 * n], layers, topk=64, W=W)
    t = res[1]["topk"][0]
    assert np.array_equal(res[2]["topk"][0], t)
    # poison every entry outside the selection (scale byte 254 = 2^127) and rerun the Reuse layer
    keep = np.zeros(n, bool)
    keep[t] = True
    pg, sl = cache.slots(0, np.nonzero(~keep)[0])
    o_before = res[2]["o"][0]
    cache.lat_scales[pg, sl] = 254
    rows = gather_rows(cache, 0, t, layers[2]["swa"][0], 2 * n - 1, W)
    o_after, _ = sparse_attention(layers[2]["q"][0], rows, 1 / math.sqrt(512))
    assert np.array_equal(o_before, o_after)


def test_decode_ignores_future_entries_and_window_rows():
    rng = np.random.default_rng(3)
    n = 700
    cache = _rand_cache(rng, n + 40)              # 40 entries beyond the context
    W, H = 128, 2
    L = 2 * n
    spec = dict(mode="full", pool_blocks=0, q=bits(rng.standard_normal((1, H, 512))),
                q_idx=bits(rng.standard_normal((1, 4, 64))), w_idx=bits(rng.standard_normal((1, 4))),
                swa=bits(rng.standard_normal((1, W, 512))))
    r1 = run_decode(cache, [L], [spec], topk=32, W=W)
    pg, sl = cache.slots(0, np.arange(n, n + 40))
    cache.idx_scales[pg, sl] = 200                # future keys become huge
    cache.lat_scales[pg, sl] = 200
    r2 = run_decode(cache, [L], [spec], topk=32, W=W)
    assert np.array_equal(r1[0]["o"][0], r2[0]["o"][0])
    assert np.array_equal(r1[0]["topk"][0], r2[0]["topk"][0])
    assert n_visible(L - 1) == n


def test_prefill_query_ignores_later_chunk_tokens():
    rng = np.random.default_rng(4)
    prior, C, W, H = 300, 20, 16, 2
    n_total = (prior + C) // 2
    cache = _rand_cache(rng, n_total)
    q = bits(rng.standard_normal((1, C, H, 512)))
    qi = bits(rng.standard_normal((1, C, 4, 64)))
    wi = bits(rng.standard_normal((1, C, 4)))
    local = bits(rng.standard_normal((1, W - 1 + C, 512)))
    i = 7                                          # query at t = prior + 7 sees entries < 154
    r1 = run_prefill(cache, [prior], C, q, qi, wi, local, topk=40, W=W, queries=[(0, i)])
    pg, sl = cache.slots(0, np.arange(n_visible(prior + i), n_total))
    cache.lat_scales[pg, sl] = 250
    cache.idx_scales[pg, sl] = 250
    local2 = local.copy()
    local2[0, W - 1 + i + 1:] = bits(np.full((C - i - 1, 512), 1000.0))
    r2 = run_prefill(cache, [prior], C, q, qi, wi, local2, topk=40, W=W, queries=[(0, i)])
    assert np.array_equal(r1[(0, i)][1], r2[(0, i)][1])
    assert np.array_equal(r1[(0, i)][0], r2[(0, i)][0])
    assert r1[(0, i)][0].max() < n_visible(prior + i)


def test_attend_on_reads_the_given_selection():
    # attend_on evaluates a layer's attention on another selection (a GPU's, which may
    # differ by near-tied scores); the returned selection stays the oracle's own
    rng = np.random.default_rng(5)
    n = 300
    cache = _rand_cache(rng, n)
    W, H, K = 16, 2, 24
    L = 2 * n
    spec = dict(mode="full", pool_blocks=0, q=bits(rng.standard_normal((1, H, 512))),
                q_idx=bits(rng.standard_normal((1, 4, 64))), w_idx=bits(rng.standard_normal((1, 4))),
                swa=bits(rng.standard_normal((1, W, 512))))
    own = run_decode(cache, [L], [spec], topk=K, W=W)
    sel = own[0]["topk"][0]
    same = run_decode(cache, [L], [spec], topk=K, W=W, attend_on=[{0: sel}])
    assert np.array_equal(same[0]["o"][0], own[0]["o"][0])
    # swap the last selected entry for one outside the selection
    other = np.sort(np.concatenate([sel[:-1], [np.setdiff1d(np.arange(n), sel)[0]]]))
    alt = run_decode(cache, [L], [spec], topk=K, W=W, attend_on=[{0: other}])
    assert np.array_equal(alt[0]["topk"][0], sel)
    rows = np.concatenate([cache.latent(0, other),
                           bf16_bits_to_f64(spec["swa"][0])[window_positions(L - 1, W) % W]])
    dense = _dense_attention_loops(bf16_bits_to_f64(spec["q"][0]), rows, 1 / math.sqrt(512))
    assert np.allclose(alt[0]["o"][0], dense, rtol=1e-12, atol=1e-12)
    assert not np.allclose(alt[0]["o"][0], own[0]["o"][0], rtol=0, atol=1e-9)
    # chunked prefill: the same option per query
    prior, C = 200, 6
    q = bits(rng.standard_normal((1, C, H, 512)))
    qi = bits(rng.standard_normal((1, C, 4, 64)))
    wi = bits(rng.standard_normal((1, C, 4)))
    local = bits(rng.standard_normal((1, W - 1 + C, 512)))
    r1 = run_prefill(cache, [prior], C, q, qi, wi, local, topk=K, W=W, queries=[(0, 3)])
    tk = r1[(0, 3)][0]
    swap = np.sort(np.concatenate([tk[1:], [np.setdiff1d(np.arange(n_visible(prior + 3)), tk)[-1]]]))
    r2 = run_prefill(cache, [prior], C, q, qi, wi, local, topk=K, W=W, queries=[(0, 3)],
                     attend_on={(0, 3): tk})
    r3 = run_prefill(cache, [prior], C, q, qi, wi, local, topk=K, W=W, queries=[(0, 3)],
                     attend_on={(0, 3): swap})
    assert np.array_equal(r2[(0, 3)][1], r1[(0, 3)][1])
    assert np.array_equal(r3[(0, 3)][0], tk) and not np.allclose(r3[(0, 3)][1], r1[(0, 3)][1], rtol=0, atol=1e-9)
