"""Seeded input generators (torch RNG on the chosen device).

Every draw is keyed by (config seed, tag, indices), so any sequence or layer
can be regenerated on its own.  torch's CPU and GPU generators give different
streams: a test that compares the two sides draws once and copies the tensors
to the other device.

Recipes (all bf16 values are the round-to-nearest-even image of an fp32 draw):
  * merge inputs x ~ N(0,1); merge weights from u ~ U(0,1) per channel and
    token.  "l2" weights w = u / sqrt(u_a^2 + u_b^2) over a token pair make the
    merged entry exactly N(0,1) before bf16 rounding of w (pre-built decode
    caches); "sum" weights w = u / (u_a + u_b) (chunked prefill, decode appends).
  * indexer keys, queries, indexer queries, indexer head weights, window rows:
    N(0,1).
  * heavy tail: a seeded uniform choice of round(frac * n) entries whose two
    source tokens (one at ratio 1) and indexer key are multiplied by 4 (exact in
    bf16).
  * ratio-1 (decoder) caches: one entry per token, the token's x and indexer key
    as drawn (no merge weights).
  * page tables: identity, a random permutation of all pages, or a random
    permutation of exactly the pages the batch needs ("fragmented").
  * log-uniform lengths: L = even(round(exp(U(ln lo, ln hi)))).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import torch

from .configs import (D_INDEX, D_LATENT, H_INDEX, PAGE, RATIO, DecodeConfig, PrefillConfig)


def _seed_of(seed: int, tag: str, idx: Tuple[int, ...]) -> int:
    h = hashlib.blake2b(f"{seed}|{tag}|{','.join(map(str, idx))}".encode(), digest_size=8)
    return int.from_bytes(h.digest(), "little") & ((1 << 63) - 1)


class Gen:
    """Keyed torch generator factory on one device."""

    def __init__(self, seed: int, device: str | torch.device = "cpu"):
        self.seed = int(seed)
        self.device = torch.device(device)

    def g(self, tag: str, *idx: int) -> torch.Generator:
        gen = torch.Generator(device=self.device)
        gen.manual_seed(_seed_of(self.seed, tag, idx))
        return gen

    def normal(self, shape, tag: str, *idx: int) -> torch.Tensor:
        return torch.randn(*shape, generator=self.g(tag, *idx), device=self.device, dtype=torch.float32)

    def normal_bf16(self, shape, tag: str, *idx: int) -> torch.Tensor:
        return self.normal(shape, tag, *idx).to(torch.bfloat16)

    def uniform(self, shape, tag: str, *idx: int) -> torch.Tensor:
        return torch.rand(*shape, generator=self.g(tag, *idx), device=self.device, dtype=torch.float32)

    def randperm(self, n: int, tag: str, *idx: int) -> torch.Tensor:
        return torch.randperm(n, generator=self.g(tag, *idx), device=self.device)

    def merge_weights(self, tokens: int, recipe: str, tag: str, *idx: int) -> torch.Tensor:
        """bf16 weights [tokens, D_LATENT] for `tokens` (even) source tokens."""
        u = self.uniform((tokens // 2, 2, D_LATENT), tag, *idx)
        u = u.clamp_min(2.0 ** -20)  # keep every pair's normaliser away from 0
        if recipe == "l2":
            den = torch.sqrt((u * u).sum(dim=1, keepdim=True))
        elif recipe == "sum":
            den = u.sum(dim=1, keepdim=True)
        else:
            raise ValueError(recipe)
        return (u / den).reshape(tokens, D_LATENT).to(torch.bfloat16)


def _log_uniform_lengths(gen: Gen, B: int, lo: int, hi: int) -> List[int]:
    u = gen.uniform((B,), "ctx_len").double().cpu()
    out = []
    for v in u.tolist():
        L = int(round(math.exp(math.log(lo) + v * (math.log(hi) - math.log(lo)))))
        L -= L % 2
        out.append(max(lo, min(hi, L)))
    return out


def _block_table(gen: Gen, kind: str, pages_per_seq: List[int]) -> Tuple[torch.Tensor, int]:
    B = len(pages_per_seq)
    mp = max(1, max(pages_per_seq))
    bt = torch.full((B, mp), -1, dtype=torch.int32)
    if kind == "identity":
        for b, n in enumerate(pages_per_seq):
            bt[b, :n] = torch.arange(b * mp, b * mp + n, dtype=torch.int32)
        return bt, B * mp
    if kind == "random":
        total = B * mp
        perm = gen.randperm(total, "pages").cpu().to(torch.int32)
        for b, n in enumerate(pages_per_seq):
            bt[b, :n] = perm[b * mp: b * mp + n]
        return bt, total
    if kind == "fragmented":
        total = sum(pages_per_seq)
        perm = gen.randperm(total, "pages").cpu().to(torch.int32)
        off = 0
        for b, n in enumerate(pages_per_seq):
            bt[b, :n] = perm[off: off + n]
            off += n
        return bt, max(total, 1)
    raise ValueError(kind)


@dataclass
class DecodeCase:
    """Inputs of one decode batch: cache build inputs, append inputs, layers."""
    cfg: DecodeConfig
    gen: Gen
    ctx_len: List[int]                 # tokens per sequence after the step's append
    prebuilt: List[int]                # tokens already in the cache before the step
    block_table: torch.Tensor          # int32 [B, max_pages] on CPU
    n_pages: int
    _layers: Dict[int, Dict[str, torch.Tensor]] = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.cfg.B

    @property
    def ratio(self) -> int:
        return self.cfg.ratio

    @property
    def n_vis(self) -> List[int]:
        return [L // self.cfg.ratio for L in self.ctx_len]

    def seq_tokens(self, b: int, recipe: str = "l2"):
        """Write inputs of the pre-built part of sequence b: x [T,512], w [T,512] (None at
        ratio 1), k_idx [T/ratio, 64]."""
        T = self.prebuilt[b]
        r = self.cfg.ratio
        x = self.gen.normal_bf16((T, D_LATENT), "x", b)
        w = self.gen.merge_weights(T, recipe, "w", b) if r == 2 else None
        k = self.gen.normal_bf16((T // r, D_INDEX), "kidx", b)
        n_heavy = int(round(self.cfg.heavy_frac * (T // r)))
        if n_heavy > 0:
            sel = self.gen.randperm(T // r, "heavy", b)[:n_heavy]
            tok = torch.cat([2 * sel, 2 * sel + 1]) if r == 2 else sel
            x[tok] = x[tok] * 4
            k[sel] = k[sel] * 4
        return x, w, k

    def append_tokens(self):
        """Tokens the step appends: x, w [B, A, 512] (w None at ratio 1), k_idx
        [B, A/ratio, 64], start_tok int32 [B]."""
        A = self.cfg.append
        r = self.cfg.ratio
        x = self.gen.normal_bf16((self.B, A, D_LATENT), "x_app")
        w = (torch.stack([self.gen.merge_weights(A, "sum", "w_app", b) for b in range(self.B)])
             if r == 2 else None)
        k = self.gen.normal_bf16((self.B, A // r, D_INDEX), "kidx_app")
        start = torch.tensor(self.prebuilt, dtype=torch.int32)
        return x, w, k, start

    def layer(self, l: int) -> Dict[str, torch.Tensor]:
        """Per-layer inputs: q [B,H,512], q_idx [B,4,64], w_idx [B,4], swa [B,W,512]."""
        if l not in self._layers:
            c = self.cfg
            self._layers[l] = dict(
                q=self.gen.normal_bf16((c.B, c.H, D_LATENT), "q", l),
                q_idx=self.gen.normal_bf16((c.B, H_INDEX, D_INDEX), "q_idx", l),
                w_idx=self.gen.normal_bf16((c.B, H_INDEX), "w_idx", l),
                swa=self.gen.normal_bf16((c.B, c.window, D_LATENT), "swa", l),
            )
        return self._layers[l]


def make_decode_case(cfg: DecodeConfig, device: str | torch.device = "cpu",
                     seed: Optional[int] = None) -> DecodeCase:
    gen = Gen(cfg.seed if seed is None else seed, device)
    if cfg.ctx is None:
        lo, hi = cfg.ctx_range
        base = _log_uniform_lengths(gen, cfg.B, lo, hi)
        ctx = [L + cfg.append for L in base]
    else:
        assert len(cfg.ctx) == cfg.B
        ctx = list(cfg.ctx)
    assert cfg.ratio in (1, 2)
    assert all(L % cfg.ratio == 0 for L in ctx) and cfg.append % cfg.ratio == 0
    prebuilt = [L - cfg.append for L in ctx]
    pages = [(L // cfg.ratio + PAGE - 1) // PAGE for L in ctx]
    bt, n_pages = _block_table(gen, cfg.pages, pages)
    return DecodeCase(cfg=cfg, gen=gen, ctx_len=ctx, prebuilt=prebuilt, block_table=bt, n_pages=n_pages)


@dataclass
class PrefillCase:
    cfg: PrefillConfig
    gen: Gen
    block_table: torch.Tensor
    n_pages: int

    @property
    def B(self) -> int:
        return self.cfg.B

    def prior_tokens(self, b: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
        T = self.cfg.prior
        return (self.gen.normal_bf16((T, D_LATENT), "x", b), self.gen.merge_weights(T, "sum", "w", b),
                self.gen.normal_bf16((T // 2, D_INDEX), "kidx", b))

    def chunk(self) -> Dict[str, torch.Tensor]:
        c = self.cfg
        W = c.window
        return dict(
            x=self.gen.normal_bf16((c.B, c.C, D_LATENT), "x_chunk"),
            w=torch.stack([self.gen.merge_weights(c.C, "sum", "w_chunk", b) for b in range(c.B)]),
            k_idx=self.gen.normal_bf16((c.B, c.C // 2, D_INDEX), "kidx_chunk"),
            q=self.gen.normal_bf16((c.B, c.C, c.H, D_LATENT), "q_chunk"),
            q_idx=self.gen.normal_bf16((c.B, c.C, H_INDEX, D_INDEX), "q_idx_chunk"),
            w_idx=self.gen.normal_bf16((c.B, c.C, H_INDEX), "w_idx_chunk"),
            local=self.gen.normal_bf16((c.B, W - 1 + c.C, D_LATENT), "local"),
            start_tok=torch.full((c.B,), c.prior, dtype=torch.int32),
        )


def make_prefill_case(cfg: PrefillConfig, device: str | torch.device = "cpu") -> PrefillCase:
    gen = Gen(cfg.seed, device)
    assert cfg.prior % 2 == 0 and cfg.C % 2 == 0
    pages = [((cfg.prior + cfg.C) // RATIO + PAGE - 1) // PAGE] * cfg.B
    bt, n_pages = _block_table(gen, cfg.pages, pages)
    return PrefillCase(cfg=cfg, gen=gen, block_table=bt, n_pages=n_pages)
