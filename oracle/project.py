"""Indexer key projected from the cache entry.  Test infrastructure.

[P1] §2.3.1: the indexer key is not stored independently of the entry; it is a
projection of the compressed main KV entry (the projection weights are trained,
so they come from the caller).  The pages give no precision for it.  Reading used
here: with y the entry's 512-d latent before quantisation (the fp32 merge of the
two tokens at ratio 2, the token itself at ratio 1) and P the caller's bf16
weights [64][512],

    k_o = fp32( s_512 ),  s_0 = 0,  s_{d+1} = fp64( s_d + P[o][d] * y[d] )  for d = 0..511

i.e. a float64 accumulation in channel order, rounded once to fp32.  Each product
of a bf16 and an fp32 value has at most 8 + 24 significant bits, so it is exact in
float64 and only the additions round; the order is part of the definition.  The
key is then quantised like any other indexer key.
"""
from __future__ import annotations

import numpy as np

D_LATENT, D_INDEX = 512, 64


def project_key_f32(y, p_vals) -> np.ndarray:
    """k [n, 64] float32 from entries y [n, 512] (fp32 values) and weights p_vals [64, 512]
    (exact bf16 values, float64): float64 accumulation over channels 0..511 in order."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    p = np.asarray(p_vals, dtype=np.float64)
    assert y.ndim == 2 and y.shape[1] == D_LATENT and p.shape == (D_INDEX, D_LATENT)
    s = np.zeros((y.shape[0], D_INDEX), dtype=np.float64)
    for d in range(D_LATENT):
        s = s + y[:, d:d + 1] * p[None, :, d]     # the product is exact; the sum rounds once
    return s.astype(np.float32)
