"""Paged FP4 cache of merged entries, as raw bytes.  Test infrastructure.

Per entry ([P1] §1.1: one shared 512-d latent for every head's key and value,
plus the indexer key; [P1] §2.3.1: the indexer key is derived from the main
entry, supplied here by the caller):
  latent  512 e2m1 codes (256 bytes, channel 2i in the low nibble) + 16 e8m0 bytes
  indexer  64 e2m1 codes ( 32 bytes)                               +  2 e8m0 bytes
Compression ratio ([P1] §2.3.1): the encoder's cache merges two tokens into one
entry (ratio 2); the decoder's cache keeps one entry per token (ratio 1, the
compressor's uncompressed special case, kept for per-token addressability), so
its write only quantises.
Entries live in pages of 64 ([P3], section on the 890-byte figure: memory is
taken in fixed blocks).  Entry j of sequence b is slot j % 64 of page
block_table[b][j // 64].  Byte arrays, one per field:
  lat_codes [n_pages][64][256], lat_scales [n_pages][64][16],
  idx_codes [n_pages][64][32],  idx_scales [n_pages][64][2].
"""
from __future__ import annotations

import numpy as np

from .fp4 import (bf16_bits_to_f64, dequantise_blocks, pack_nibbles, quantise_blocks, unpack_nibbles)
from .merge import merge_pair_f32
from .project import project_key_f32

PAGE = 64
D_LATENT = 512
D_INDEX = 64
BYTES_LATENT = D_LATENT // 2 + D_LATENT // 32      # 272
BYTES_INDEX = D_INDEX // 2 + D_INDEX // 32         # 34
BYTES_PER_ENTRY = BYTES_LATENT + BYTES_INDEX       # 306


class OracleCache:
    def __init__(self, n_pages: int, block_table, ratio: int = 2):
        assert ratio in (1, 2)
        self.ratio = int(ratio)
        self.n_pages = int(n_pages)
        self.block_table = np.asarray(block_table, dtype=np.int64)
        self.lat_codes = np.zeros((n_pages, PAGE, D_LATENT // 2), np.uint8)
        self.lat_scales = np.zeros((n_pages, PAGE, D_LATENT // 32), np.uint8)
        self.idx_codes = np.zeros((n_pages, PAGE, D_INDEX // 2), np.uint8)
        self.idx_scales = np.zeros((n_pages, PAGE, D_INDEX // 32), np.uint8)

    def slots(self, b: int, js) -> tuple[np.ndarray, np.ndarray]:
        js = np.asarray(js, dtype=np.int64)
        return self.block_table[b, js // PAGE], js % PAGE

    def write(self, b: int, start_tok: int, x_bits, w_bits, kidx_bits, chunk: int = 2048,
              latent: bool = True) -> None:
        """Store the entries of tokens start_tok .. start_tok+T-1.

        Ratio 2: merge token pairs (start_tok, start_tok+1), ... into entries
        start_tok/2 onward; x_bits, w_bits: bf16 bit patterns [T, 512]; kidx_bits:
        [T/2, 64]; T and start_tok even.  Ratio 1: entry start_tok+i is token i
        itself (w_bits unused, may be None); kidx_bits: [T, 64].  latent=False
        stores only the indexer keys (x and w unused), for checks that read the
        latent of a few entries written separately.
        """
        if self.ratio == 1:
            self._write_tokens(b, start_tok, x_bits, kidx_bits, chunk, latent)
            return
        x = np.asarray(x_bits)
        w = np.asarray(w_bits)
        k = np.asarray(kidx_bits)
        T = 2 * k.shape[0]
        assert start_tok % 2 == 0 and (not latent or x.shape[0] == T)
        for i0 in range(0, T // 2, chunk):
            i1 = min(T // 2, i0 + chunk)
            pg, sl = self.slots(b, np.arange(start_tok // 2 + i0, start_tok // 2 + i1))
            if latent:
                xs = bf16_bits_to_f64(x[2 * i0: 2 * i1])
                ws = bf16_bits_to_f64(w[2 * i0: 2 * i1])
                y = merge_pair_f32(xs[0::2], xs[1::2], ws[0::2], ws[1::2])
                lc, lu = quantise_blocks(y.astype(np.float64))
                self.lat_codes[pg, sl] = pack_nibbles(lc)
                self.lat_scales[pg, sl] = lu
            ic, iu = quantise_blocks(bf16_bits_to_f64(k[i0:i1]))
            self.idx_codes[pg, sl] = pack_nibbles(ic)
            self.idx_scales[pg, sl] = iu

    def _write_tokens(self, b: int, start_tok: int, x_bits, kidx_bits, chunk: int, latent: bool) -> None:
        """Ratio 1: quantise each token's bf16 latent and indexer key as they are."""
        k = np.asarray(kidx_bits)
        T = k.shape[0]
        x = np.asarray(x_bits) if latent else None
        assert start_tok >= 0 and (not latent or x.shape[0] == T)
        for i0 in range(0, T, chunk):
            i1 = min(T, i0 + chunk)
            pg, sl = self.slots(b, np.arange(start_tok + i0, start_tok + i1))
            if latent:
                lc, lu = quantise_blocks(bf16_bits_to_f64(x[i0:i1]))
                self.lat_codes[pg, sl] = pack_nibbles(lc)
                self.lat_scales[pg, sl] = lu
            ic, iu = quantise_blocks(bf16_bits_to_f64(k[i0:i1]))
            self.idx_codes[pg, sl] = pack_nibbles(ic)
            self.idx_scales[pg, sl] = iu

    def write_projected(self, b: int, start_tok: int, x_bits, w_bits, p_bits, chunk: int = 1024) -> None:
        """Store the entries of tokens start_tok .. start_tok+T-1 with indexer keys projected
        from the entries themselves (project.py) by the bf16 weights p_bits [64][512]
        instead of keys supplied per entry.  Ratio 2: x_bits, w_bits [T, 512], T and
        start_tok even; ratio 1: x_bits [T, 512], w_bits unused."""
        x = np.asarray(x_bits)
        p = bf16_bits_to_f64(np.asarray(p_bits))
        r = self.ratio
        T = x.shape[0]
        assert T % r == 0 and start_tok % r == 0
        n = T // r
        for i0 in range(0, n, chunk):
            i1 = min(n, i0 + chunk)
            pg, sl = self.slots(b, np.arange(start_tok // r + i0, start_tok // r + i1))
            if r == 2:
                xs = bf16_bits_to_f64(x[2 * i0: 2 * i1])
                ws = bf16_bits_to_f64(np.asarray(w_bits)[2 * i0: 2 * i1])
                y = merge_pair_f32(xs[0::2], xs[1::2], ws[0::2], ws[1::2])
            else:
                y = bf16_bits_to_f64(x[i0:i1]).astype(np.float32)
            lc, lu = quantise_blocks(y.astype(np.float64))
            self.lat_codes[pg, sl] = pack_nibbles(lc)
            self.lat_scales[pg, sl] = lu
            ic, iu = quantise_blocks(project_key_f32(y, p).astype(np.float64))
            self.idx_codes[pg, sl] = pack_nibbles(ic)
            self.idx_scales[pg, sl] = iu

    def latent(self, b: int, js) -> np.ndarray:
        """Dequantised latent rows [len(js), 512] (float64)."""
        pg, sl = self.slots(b, js)
        return dequantise_blocks(unpack_nibbles(self.lat_codes[pg, sl]), self.lat_scales[pg, sl])

    def index_keys(self, b: int, js) -> np.ndarray:
        """Dequantised indexer keys [len(js), 64] (float64)."""
        pg, sl = self.slots(b, js)
        return dequantise_blocks(unpack_nibbles(self.idx_codes[pg, sl]), self.idx_scales[pg, sl])
