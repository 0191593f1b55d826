"""Pins of the oracle's projected indexer key (oracle/project.py) and of the cache
write that uses it: closed forms, the exact sum, the defined accumulation order, and
agreement with the write path that takes the key from the caller."""
from fractions import Fraction

import numpy as np

from oracle import (OracleCache, bf16_bits_to_f64, f64_to_bf16_bits, merge_pair_f32, project_key_f32,
                    quantise_blocks, pack_nibbles)


def _bf16(x):
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def _f32_nearest(q: Fraction) -> np.float32:
    """Exact rational -> nearest float32 (ties to even), without double rounding."""
    f = np.float32(float(q))                      # within one fp32 ulp of q
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_selection_weights_give_the_channels():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((50, 512)).astype(np.float32) * np.float32(3.0)
    perm = rng.permutation(512)[:64]
    p = np.zeros((64, 512))
    p[np.arange(64), perm] = 1.0
    assert np.array_equal(project_key_f32(y, p), y[:, perm])


def test_power_of_two_single_weights_scale_exactly():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((30, 512)).astype(np.float32)
    perm = rng.permutation(512)[:64]
    a = rng.integers(-20, 21, size=64)
    p = np.zeros((64, 512))
    p[np.arange(64), perm] = np.ldexp(1.0, a)
    want = (y[:, perm].astype(np.float64) * np.ldexp(1.0, a)[None, :]).astype(np.float32)
    assert np.array_equal(project_key_f32(y, p), want)


def test_matches_the_exact_sum_within_one_ulp():
    # A dropped or repeated term, a sign error or a transposed weight index moves the
    # result far beyond one fp32 ulp; the float64 accumulation itself stays within it.
    rng = np.random.default_rng(3)
    y = rng.standard_normal((6, 512)).astype(np.float32)
    p = _bf16(rng.standard_normal((64, 512)) / np.sqrt(512))
    got = project_key_f32(y, p)
    same = 0
    for n in range(y.shape[0]):
        for o in range(64):
            exact = sum((Fraction(float(p[o, d])) * Fraction(float(y[n, d])) for d in range(512)), Fraction(0))
            want = _f32_nearest(exact)
            g = got[n, o]
            assert g == want or np.nextafter(want, np.float32(np.inf)) == g or np.nextafter(want, np.float32(-np.inf)) == g
            same += int(g == want)
    assert same >= 0.99 * y.shape[0] * 64


def test_accumulation_runs_in_channel_order():
    # 2^60 + 1 rounds to 2^60 in float64, so channel order 0, 1, 2 gives 0 where the
    # exact sum is 1: the defined order, not the exact value, decides the key.
    y = np.zeros((1, 512), np.float32)
    y[0, :3] = [2.0 ** 60, 1.0, -2.0 ** 60]
    p = np.zeros((64, 512))
    p[0, :3] = 1.0
    p[1, 1] = 1.0
    k = project_key_f32(y, p)
    assert k[0, 0] == 0.0 and k[0, 1] == 1.0


def test_projected_write_equals_the_supplied_key_write():
    # With weights that select channels 0..63, the projected key of a ratio-1 entry is
    # the token's first 64 channels, so the bytes equal those of the write that takes
    # that key from the caller; at ratio 2 it is the merged entry's first 64 channels.
    rng = np.random.default_rng(4)
    sel = np.zeros((64, 512), np.uint16)
    sel[np.arange(64), np.arange(64)] = f64_to_bf16_bits(1.0)
    bt = np.array([[2, 0, 1]])
    x = f64_to_bf16_bits(rng.standard_normal((130, 512)) * 2.0)
    a, b = OracleCache(3, bt, ratio=1), OracleCache(3, bt, ratio=1)
    a.write_projected(0, 4, x, None, sel)
    b.write(0, 4, x, None, x[:, :64])
    for f in ("lat_codes", "lat_scales", "idx_codes", "idx_scales"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    w = f64_to_bf16_bits(rng.uniform(0, 1, (130, 512)))
    c = OracleCache(3, bt, ratio=2)
    c.write_projected(0, 2, x, w, sel)
    xs, ws = bf16_bits_to_f64(x), bf16_bits_to_f64(w)
    y = merge_pair_f32(xs[0::2], xs[1::2], ws[0::2], ws[1::2])
    ic, iu = quantise_blocks(y[:, :64].astype(np.float64))
    pg, sl = c.slots(0, np.arange(1, 66))
    assert np.array_equal(c.idx_codes[pg, sl], pack_nibbles(ic))
    assert np.array_equal(c.idx_scales[pg, sl], iu)
    lc, lu = quantise_blocks(y.astype(np.float64))
    assert np.array_equal(c.lat_codes[pg, sl], pack_nibbles(lc))
