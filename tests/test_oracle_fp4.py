"""Pins of the oracle's FP4 format, quantiser and bf16 rounding (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (E2M1_VALUES, bf16_bits_to_f64, dequantise_blocks, e2m1_decode, e8m0_decode,
                    f64_to_bf16_bits, pack_nibbles, quantise_blocks, unpack_nibbles)


def _e2m1_from_bitfields(c: int) -> float:
    """OCP e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    mag = (2.0 ** (e - 1)) * (1 + m / 2) if e > 0 else m / 2
    return -mag if s else mag


def test_e2m1_code_table_matches_bitfield_definition():
    for c in range(16):
        got = float(e2m1_decode(np.array([c]))[0])
        want = _e2m1_from_bitfields(c)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c


def test_e8m0_every_byte():
    u = np.arange(256)
    s = e8m0_decode(u)
    for k in range(255):
        assert s[k] == Fraction(2) ** (k - 127)
    assert np.isnan(s[255])


def test_exhaustive_codes_round_trip_when_block_max_is_4_or_6():
    rng = np.random.default_rng(0)
    for u in [0, 1, 2, 60, 125, 127, 128, 200, 252]:
        for top in (6, 7, 14, 15):              # magnitude 4 or 6, either sign
            for trial in range(20):
                codes = rng.integers(0, 16, size=32).astype(np.uint8)
                codes[trial % 32] = top
                codes = np.where((codes & 7) > 5, np.uint8(top), codes)  # keep the top magnitude the max
                v = dequantise_blocks(codes, np.array([u], np.uint8))
                c2, u2 = quantise_blocks(v)
                assert int(u2[0]) == u
                assert np.array_equal(c2, codes), (u, codes, c2)


def test_every_code_at_every_scale_decodes_to_value_times_power_of_two():
    for u in range(255):
        codes = np.arange(32, dtype=np.uint8) % 16
        v = dequantise_blocks(codes, np.array([u], np.uint8))
        for c, x in zip(codes, v):
            assert Fraction(x) == Fraction(_e2m1_from_bitfields(int(c))) * Fraction(2) ** (u - 127)


def test_ties_go_to_even_code_and_saturation():
    # block max 5 -> floor(log2 5) - 2 = 0, so the scaled values are the inputs themselves
    v = np.array([5.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -0.25, -0.75, 0.2, 0.3, 2.4, 2.6, 3.4, 3.6,
                  4.9, 5.1, 0.0, -0.0, 1.0, 1.5, 2.0, 3.0, 4.0, -5.0, -1.25, -3.5, 0.74, 0.76, 1.26,
                  1.74, 1.76])
    want = np.array([4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, -0.0, -1.0, 0.0, 0.5, 2.0, 3.0, 3.0, 4.0,
                     4.0, 6.0, 0.0, -0.0, 1.0, 1.5, 2.0, 3.0, 4.0, -4.0, -1.0, -4.0, 0.5, 1.0, 1.5,
                     1.5, 2.0])
    c, u = quantise_blocks(v)
    assert u[0] == 127
    got = dequantise_blocks(c, u)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(v))
    # values between 6 and 8 times the scale saturate to 6
    c, u = quantise_blocks(np.array([7.9] + [0.0] * 31))
    assert u[0] == 127 and dequantise_blocks(c, u)[0] == 6.0


def test_quantised_value_is_a_nearest_grid_point():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((400, 32)) * np.ldexp(1.0, rng.integers(-30, 30, size=(400, 1)))
    v = v.astype(np.float32).astype(np.float64)
    c, u = quantise_blocks(v)
    vq = dequantise_blocks(c, u)
    scale = e8m0_decode(u)[:, None]
    grid = np.concatenate([-E2M1_VALUES[::-1], E2M1_VALUES])
    for i in range(v.shape[0]):
        for j in range(32):
            d_best = np.min(np.abs(v[i, j] - grid * scale[i, 0]))
            assert abs(v[i, j] - vq[i, j]) == d_best
    # the scale follows floor(log2 amax) - 2
    amax = np.abs(v).max(axis=1)
    assert np.array_equal(u[:, 0].astype(int) - 127, np.floor(np.log2(amax)).astype(int) - 2)


def test_heavy_tail_times_4_keeps_codes_and_adds_2_to_scale():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((100, 512)).astype(np.float32).astype(np.float64)
    c1, u1 = quantise_blocks(v)
    c4, u4 = quantise_blocks(v * 4)
    assert np.array_equal(c1, c4)
    assert np.array_equal(u4.astype(int), u1.astype(int) + 2)


def test_zero_block_and_extreme_scales():
    c, u = quantise_blocks(np.array([0.0, -0.0] * 16))
    assert u[0] == 0 and not c.any()
    c, u = quantise_blocks(np.array([2.0 ** -140] + [0.0] * 31))
    assert u[0] == 0 and dequantise_blocks(c, u)[0] == 0.0
    big = float(np.float32(2.0 ** 127 * 1.5))
    c, u = quantise_blocks(np.array([big] + [1.0] * 31))
    assert u[0] == 127 + 125 and dequantise_blocks(c, u)[0] == big


def test_nibble_packing_low_nibble_is_even_channel():
    codes = np.arange(16, dtype=np.uint8)
    p = pack_nibbles(codes)
    assert list(p) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(unpack_nibbles(p), codes)


def test_bf16_rounding_matches_torch_for_fp32_values_and_ties():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.ldexp(1.0, rng.integers(-140, 120, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, want)
    # exact ties: 1 + 2^-8 -> 1 (even); 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert bf16_bits_to_f64(f64_to_bf16_bits(np.array([1 + 2.0 ** -8]))) == 1.0
    assert bf16_bits_to_f64(f64_to_bf16_bits(np.array([1 + 3 * 2.0 ** -8]))) == 1 + 2.0 ** -6
    # a float64 value just above a bf16 tie rounds up (no double rounding through fp32)
    assert bf16_bits_to_f64(f64_to_bf16_bits(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))) == 1 + 2.0 ** -7
