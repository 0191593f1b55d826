"""Workload shapes of the five CSA2 decode / prefill configurations.

Fixed sizes follow the CSA2 description in "DeepSeek-v4.1 Flash:
KVキャッシュ圧縮の限界を押し広げる" (hackernews.jp, zartbot's walk-through):
512-d shared latent (§1.1, §1.2), sliding window 128 (§1.2), top-K 512 and
HSI candidate blocks of 8 positions (§2.3.4), pairwise merge in the encoder
(§1.1, §2.3.1).  Head count, indexer size and batch shapes are the workload's
own choices (the page leaves them blank).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

D_LATENT = 512      # shared latent width
D_INDEX = 64        # indexer key / query width per head
H_INDEX = 4         # indexer heads
TOPK = 512          # entries read per query
WINDOW = 128        # sliding-window tokens
CAND_BLOCK = 8      # HSI candidate block (positions per block)
PAGE = 64           # entries per cache page
RATIO = 2           # tokens merged into one entry (encoder)


@dataclass(frozen=True)
class LayerSpec:
    """One CSA2 layer of a decode schedule.

    mode: "full" | "reindex" | "reuse".  pool_blocks: candidate-pool blocks a
    Full layer keeps for later Reindex layers (0 = no pool).
    """
    mode: str
    pool_blocks: int = 0


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    ctx: Tuple[int, ...] | None          # tokens per sequence (None: drawn log-uniform)
    layers: Tuple[LayerSpec, ...]
    pages: str = "identity"             # identity | random | fragmented
    heavy_frac: float = 0.0             # fraction of entries scaled x4 before quantisation
    append: int = 0                     # tokens written by the step before decoding
    ctx_range: Tuple[int, int] | None = None   # log-uniform bounds when ctx is None
    topk: int = TOPK
    window: int = WINDOW
    cand_block: int = CAND_BLOCK
    seed: int = 1000
    ratio: int = RATIO                 # tokens per entry: 2 (encoder) or 1 (decoder)

    @property
    def n_layers(self) -> int:
        return len(self.layers)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    prior: int          # tokens already cached before the chunk
    C: int              # query tokens in the chunk
    topk: int = TOPK
    window: int = WINDOW
    pages: str = "identity"
    seed: int = 1003


FULL = LayerSpec("full")

# The pages' schedules ([P1] §2.3.3): the decoder runs a Full block ([Full + 3 Reuse],
# the Full layer keeping the 2048-block HSI pool of §2.3.4) and four Reindex blocks
# ([Reindex + 3 Reuse]); an encoder block is [Full + 5 Reuse], three of them.
DECODER_SCHEDULE = ((LayerSpec("full", 2048),) + (LayerSpec("reuse"),) * 3 +
                    ((LayerSpec("reindex"),) + (LayerSpec("reuse"),) * 3) * 4)
ENCODER_SCHEDULE = ((LayerSpec("full"),) + (LayerSpec("reuse"),) * 5) * 3

CONFIGS = {
    0: DecodeConfig("c0_b1_ctx2k_h16_full", B=1, H=16, ctx=(2048,),
                    layers=(LayerSpec("full", 256),), seed=1000),
    1: DecodeConfig("c1_b32_ctx64k_h64_full_reindex_reuse", B=32, H=64, ctx=(65536,) * 32,
                    layers=(LayerSpec("full", 512), LayerSpec("reindex"), LayerSpec("reuse")),
                    heavy_frac=0.05, seed=1001),
    2: DecodeConfig("c2_b8_ctx1m_h64_full_randpages", B=8, H=64, ctx=(1048576,) * 8,
                    layers=(LayerSpec("full", 0),), pages="random", seed=1002),
    3: PrefillConfig("c3_prefill_b4_prior128k_c4096_h64", B=4, H=64, prior=131072, C=4096,
                     seed=1003),
    4: DecodeConfig("c4_b128_ctx1k_256k_h64_mixed", B=128, H=64, ctx=None, ctx_range=(1024, 262144),
                    layers=(LayerSpec("full", 512), LayerSpec("reuse"), LayerSpec("reindex"),
                            LayerSpec("reuse")),
                    pages="fragmented", append=64, seed=1004),
    # The decoder's ratio-1 cache (one entry per token) with the pages' HSI setting of
    # 2048 candidate blocks of 8 positions (16384 candidates); 32K tokens per sequence
    # give the same 32768 entries as config 1.
    5: DecodeConfig("c5_b32_ctx32k_h64_ratio1_pool2048", B=32, H=64, ctx=(32768,) * 32,
                    layers=(LayerSpec("full", 2048), LayerSpec("reindex"), LayerSpec("reuse")),
                    heavy_frac=0.05, seed=1005, ratio=1),
}


def small_decode(base: int, B: int, ctx: Tuple[int, ...] | None = None, H: int | None = None,
                 seed: int | None = None, **kw) -> DecodeConfig:
    """A reduced copy of decode config `base` that the oracle finishes in seconds."""
    c = CONFIGS[base]
    assert isinstance(c, DecodeConfig)
    if ctx is None and c.ctx is None:
        ctx_range = kw.pop("ctx_range", (256, 20000))
    else:
        ctx_range = kw.pop("ctx_range", c.ctx_range)
    return DecodeConfig(
        name=f"{c.name}_small", B=B, H=H if H is not None else c.H, ctx=ctx, layers=kw.pop("layers", c.layers),
        pages=kw.pop("pages", c.pages), heavy_frac=kw.pop("heavy_frac", c.heavy_frac),
        append=kw.pop("append", c.append), ctx_range=ctx_range, topk=kw.pop("topk", c.topk),
        window=kw.pop("window", c.window), cand_block=kw.pop("cand_block", c.cand_block),
        seed=seed if seed is not None else c.seed + 100, ratio=kw.pop("ratio", c.ratio))


def small_prefill(B: int = 2, prior: int = 3000, C: int = 96, H: int = 16, seed: int = 1103,
                  **kw) -> PrefillConfig:
    return PrefillConfig(name="c3_prefill_small", B=B, H=H, prior=prior, C=C, seed=seed, **kw)
