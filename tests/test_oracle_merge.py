"""Pins of the oracle's pairwise merge and cache layout (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (BYTES_INDEX, BYTES_LATENT, BYTES_PER_ENTRY, OracleCache, bf16_bits_to_f64,
                    merge_pair_f32, quantise_blocks)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def _fp32_rne(r: Fraction) -> float:
    """Round a rational to fp32 (nearest, ties to even), by exact rational arithmetic."""
    if r == 0:
        return 0.0
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q_exp = max(e - 23, -149)                     # 24 significant bits; subnormal spacing 2^-149
    q = a / Fraction(2) ** q_exp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = Fraction(n) * Fraction(2) ** q_exp
    if v >= Fraction(2) ** 128:
        return sign * float("inf")
    return sign * float(v)


def _rand_bf16(rng, n, lo, hi):
    m = rng.integers(128, 256, size=n)            # 8 significant bits
    e = rng.integers(lo, hi, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return s * np.ldexp(m.astype(np.float64), e - 7)


def test_merge_rounds_once_like_exact_rational_sum():
    rng = np.random.default_rng(0)
    n = 4000
    x0, x1 = _rand_bf16(rng, n, -60, 60), _rand_bf16(rng, n, -60, 60)
    w0, w1 = _rand_bf16(rng, n, -60, 10), _rand_bf16(rng, n, -60, 10)
    y = merge_pair_f32(x0, x1, w0, w1)
    for i in range(n):
        exact = Fraction(w0[i]) * Fraction(x0[i]) + Fraction(w1[i]) * Fraction(x1[i])
        assert float(y[i]) == _fp32_rne(exact), i


def test_merge_closed_forms():
    rng = np.random.default_rng(1)
    x0 = rng.standard_normal((64, 512)).astype(np.float32).astype(np.float64)
    x1 = rng.standard_normal((64, 512)).astype(np.float32).astype(np.float64)
    # w = (1, 0): the entry is the even token
    y = merge_pair_f32(x0, x1, np.ones_like(x0), np.zeros_like(x0))
    assert np.array_equal(y.astype(np.float64), x0)
    c_a, u_a = quantise_blocks(y.astype(np.float64))
    c_b, u_b = quantise_blocks(x0)
    assert np.array_equal(c_a, c_b) and np.array_equal(u_a, u_b)
    # w = (1/2, 1/2): the fp32-rounded exact mean
    y = merge_pair_f32(x0, x1, np.full_like(x0, 0.5), np.full_like(x0, 0.5))
    assert np.array_equal(y, ((x0 + x1) / 2).astype(np.float32))


def test_bytes_per_entry_and_page_count_against_pages():
    assert BYTES_LATENT == 272 and BYTES_INDEX == 34 and BYTES_PER_ENTRY == 306
    ratio = GOLDEN["encoder_merge_ratio"]["value"]
    copies = GOLDEN["cache_copies"]
    per_token_encoder = BYTES_PER_ENTRY / ratio                      # 153 B per token per copy
    per_token = copies["encoder"] * per_token_encoder + copies["decoder"] * BYTES_PER_ENTRY
    # This format gives 765 B/token under the pages' 3 + 1 copies, not the printed ~890:
    # the pages do not give their layout (documented mismatch).
    assert per_token == 765
    assert abs(per_token - GOLDEN["bytes_per_token_global_kv_plus_indexer"]["value"]) / 890 < 0.15
    # 2048 tokens -> 1024 entries
    assert 2048 // ratio == 1024


def test_cache_write_layout_and_paging():
    rng = np.random.default_rng(2)
    T = 2 * 150
    bt = np.array([[3, 0, 2]])
    cache = OracleCache(4, bt)
    xb = (rng.integers(0, 2 ** 15, size=(T, 512)) & 0x3FFF | 0x3C00).astype(np.uint16)  # |x| in [2^-7, 2)
    wb = np.full((T, 512), 0x3F80, np.uint16)                                           # w = 1
    wb[1::2] = 0                                                                        # odd tokens ignored
    kb = (rng.integers(0, 2 ** 15, size=(T // 2, 64)) & 0x3FFF | 0x3C00).astype(np.uint16)
    cache.write(0, 20, xb, wb, kb)
    # entry 10 + i sits in page bt[(10+i)//64], slot (10+i)%64 and equals quantise(x_{2i})
    for i in [0, 1, 53, 54, 117, 149]:
        j = 10 + i
        pg, sl = bt[0, j // 64], j % 64
        c, u = quantise_blocks(bf16_bits_to_f64(xb[2 * i]))
        packed = (c[0::2] | (c[1::2] << 4)).astype(np.uint8)
        assert np.array_equal(cache.lat_codes[pg, sl], packed)
        assert np.array_equal(cache.lat_scales[pg, sl], u)
        ck, uk = quantise_blocks(bf16_bits_to_f64(kb[i]))
        assert np.array_equal(cache.idx_codes[pg, sl], (ck[0::2] | (ck[1::2] << 4)).astype(np.uint8))
        assert np.array_equal(cache.idx_scales[pg, sl], uk)
    # nothing written before entry 10 or in the unused page
    assert not cache.lat_codes[3, :10].any() and not cache.lat_codes[1].any()
