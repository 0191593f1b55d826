"""Sparse attention over the selected entries plus the sliding window.  Test infrastructure.

[P1] §2.3.1: each query attends at once to the selected global entries and to
the layer's local sliding-window KV; [P1] §1.2: window 128, a 512-d latent
shared by all query heads (used here as both key and value).  [P3]
("計算としては、照合して、重みをつけて、足し合わせる"): dot the query with each key,
turn the scores into weights that sum to 1, add the values with those weights.
[P3] ("未来を見ずに、続きを予測する"): position t sees itself and the past only.

Readings: one softmax over global and window rows together, scale 1/sqrt(512),
no sink or bias, the window holds positions max(0, t-W+1)..t in ring slot
pos % W, no de-duplication between window rows and merged entries.
"""
from __future__ import annotations

import numpy as np

from .fp4 import bf16_bits_to_f64


def window_positions(t: int, W: int) -> np.ndarray:
    return np.arange(max(0, t - W + 1), t + 1)


def gather_rows(cache, b: int, topk_ids, swa_bits, t: int, W: int) -> np.ndarray:
    """Rows the query at position t reads: dequantised selected entries, then window rows."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    ids = ids[ids >= 0]
    lat = cache.latent(b, ids) if ids.size else np.zeros((0, 512))
    swa = bf16_bits_to_f64(np.asarray(swa_bits))
    win = swa[window_positions(t, W) % W]
    return np.concatenate([lat, win], axis=0)


def sparse_attention(q_bits, rows, sm_scale: float):
    """o_h = softmax(sm_scale * q_h . R^T) R for every head; returns (o [H,512], lse [H]) in float64."""
    q = bf16_bits_to_f64(q_bits)
    rows = np.asarray(rows, dtype=np.float64)
    z = sm_scale * (q @ rows.T)                          # [H, R]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ rows) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse
