"""Pairwise merge of two adjacent positions into one cache entry.  Test infrastructure.

[P1] §1.1 (sequence dimension) and [P2] ("CSA2：3次元同時圧縮..."): the
encoder merges two adjacent positions into one cache entry with learned
per-channel weights; [P1] §2.3.1 adds that CSA2's compressor has no window
overlap and no absolute position embedding.  Reading used: per token and per
channel bf16 weights from the caller, entry_c = w_{2j,c} x_{2j,c} +
w_{2j+1,c} x_{2j+1,c}, no normalisation, rounded once to fp32.
"""
from __future__ import annotations

import numpy as np


def merge_pair_f32(x0, x1, w0, w1) -> np.ndarray:
    """fp32 round-to-nearest-even of w0*x0 + w1*x1, computed exactly before the one rounding.

    Inputs are the exact values of bf16 numbers (float64 arrays).  Products of
    two bf16 values are exact in float64; the float64 sum is exact unless the
    two terms are more than ~37 binades apart, so its rounding error is
    recovered with TwoSum and used to settle the fp32 rounding when the float64
    sum lands exactly on an fp32 halfway point.
    """
    p0 = np.asarray(w0, np.float64) * np.asarray(x0, np.float64)
    p1 = np.asarray(w1, np.float64) * np.asarray(x1, np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        s = p0 + p1
        bb = s - p0
        err = (p0 - (s - bb)) + (p1 - bb)            # exact: p0 + p1 = s + err
        err = np.where(np.isfinite(s), err, 0.0)
        y = s.astype(np.float32)                      # correct unless s sits on a halfway point
        yd = y.astype(np.float64)
        toward = np.where(s > yd, np.float32(np.inf), np.float32(-np.inf))
        nb = np.nextafter(y, toward)
        mid = (yd + nb.astype(np.float64)) / 2
        on_half = np.isfinite(s) & (s != yd) & (s == mid) & (err != 0)
        # the exact value lies strictly on err's side of the halfway point
        fix = np.where((err > 0) == (nb > y), nb, y)
        y = np.where(on_half, fix, y)
    return y.astype(np.float32)
