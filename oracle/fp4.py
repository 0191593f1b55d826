"""FP4 (e2m1) values with one e8m0 power-of-two scale per 32 values.  Test infrastructure.

[P1] §1.1 and [P2] ("CSA2：3次元同時圧縮...") say the global KV and the
indexer keys are stored in FP4; [P3] (section on making the record smaller:
"小さくする方法は、「メモのどこを減らすか」で分ける") adds that FP4 holds the
base value in 4 bits plus auxiliary data that adjusts magnitude.  The pages
give no block format.  Reading used here (the workload's MXFP4 format):
e2m1 codes, one e8m0 scale byte per block of 32 consecutive channels,
scale exponent = floor(log2(max|v|)) - 2, round to nearest with ties to the
even code, saturate at 6, keep the sign bit, all-zero block -> scale byte 0.
"""
from __future__ import annotations

import numpy as np

# e2m1 magnitudes indexed by the 3 low bits of the code; bit 3 is the sign.
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
MX_BLOCK = 32
E2M1_EMAX = 2          # exponent of the largest e2m1 magnitude (6 = 1.5 * 2^2)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 numbers given as raw uint16 bit patterns."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) in one step; return bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # |xf| = m * 2^e, m in [0.5, 1)
    # bf16 keeps 8 significant bits; below 2^-126 the spacing stays 2^-133.
    q_exp = np.maximum(e - 8, -133)
    quantum = np.ldexp(1.0, q_exp)
    r = np.rint(xf / quantum) * quantum       # rint: round half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xf), r)
    out[...] = np.where(finite, r, x)
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def e2m1_decode(codes) -> np.ndarray:
    """Value of 4-bit e2m1 codes (bit 3 = sign)."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e8m0_decode(u) -> np.ndarray:
    """Scale 2^(u-127) of an e8m0 byte; 255 is NaN (never produced by quantise_blocks)."""
    u = np.asarray(u).astype(np.int64)
    s = np.ldexp(1.0, u - 127)
    return np.where(u == 255, np.nan, s)


def _nearest_code_magnitude(x: np.ndarray) -> np.ndarray:
    """Index into E2M1_VALUES of the grid point nearest to x >= 0; a tie goes to the even index."""
    d = np.abs(x[..., None] - E2M1_VALUES)            # distance to each grid point
    best = d.min(axis=-1, keepdims=True)
    is_best = d == best
    idx = np.argmax(is_best, axis=-1)                 # first (lower) nearest point
    upper = np.minimum(idx + 1, 7)
    tie = np.take_along_axis(is_best, upper[..., None], axis=-1)[..., 0] & (upper != idx)
    # on a tie between idx and idx+1 take whichever index is even
    return np.where(tie & (idx % 2 == 1), upper, idx)


def quantise_blocks(v) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 values (last axis a multiple of 32) to e2m1 codes + e8m0 scale bytes.

    Returns (codes uint8 [..., n] with values 0..15, scales uint8 [..., n/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    assert v.shape[-1] % MX_BLOCK == 0
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    floor_log2 = ex - 1
    e = np.clip(floor_log2 - E2M1_EMAX, -127, 127)
    e = np.where(amax == 0, -127, e)
    u = (e + 127).astype(np.uint8)
    scaled = np.abs(blocks) / np.ldexp(1.0, e)[..., None]
    mag = _nearest_code_magnitude(np.minimum(scaled, 8.0))   # beyond 6 the nearest point is 6
    sign = np.signbit(blocks).astype(np.int64)
    codes = (mag | (sign << 3)).astype(np.uint8)
    codes = np.where((amax == 0)[..., None], np.uint8(0), codes)
    return codes.reshape(v.shape), u


def dequantise_blocks(codes, u) -> np.ndarray:
    """Values e2m1(code) * 2^(u-127), block scale shared by 32 consecutive codes."""
    codes = np.asarray(codes)
    vals = e2m1_decode(codes)
    n = codes.shape[-1]
    vals = vals.reshape(codes.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    return (vals * e8m0_decode(u)[..., None]).reshape(codes.shape)


def pack_nibbles(codes) -> np.ndarray:
    """Two codes per byte: channel 2i in the low nibble, channel 2i+1 in the high nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed) -> np.ndarray:
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out
