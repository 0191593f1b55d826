"""CPU oracle for CSA2 compressed-KV sparse decode.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or run anything in this package.  The HIP product path never calls it
and shares no code, tables or helpers with it.

Plain NumPy in float64: slow, direct, one step per definition.  Sources
(web pages on DeepSeek-V4.1 Flash and its CSA2 attention):
  [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる"
       (hackernews.jp translation of zartbot's walk-through of the tech report)
  [P2] ai.freelance-job.com news summary of the same article
       (spec table "モデルの基本スペック"; "CSA2：3次元同時圧縮でKVをさらに削る")
  [P3] "DeepSeek V4.1 Flash architecture: making a giant AI faster through reuse"
       (yasmorita.com)
Where the pages are silent (FP4 block format, score formula, rounding, tie
order), the workload's stated reading is followed; each such function says so.

Parity pins: every function here is pinned by tests in tests/test_oracle_*.py
against closed forms, brute force, invariants or numbers the pages print.
"""
from .fp4 import (E2M1_VALUES, bf16_bits_to_f64, f64_to_bf16_bits, e2m1_decode, e8m0_decode,
                  quantise_blocks, dequantise_blocks, pack_nibbles, unpack_nibbles)
from .merge import merge_pair_f32
from .project import project_key_f32
from .cache import OracleCache, BYTES_LATENT, BYTES_INDEX, BYTES_PER_ENTRY
from .indexer import (index_scores, topk_select, hsi_pool, full_layer, reindex_layer)
from .hisa import block_summaries, hisa_layer
from .attention import sparse_attention, gather_rows
from .schedule import run_decode, run_prefill

__all__ = [
    "E2M1_VALUES", "bf16_bits_to_f64", "f64_to_bf16_bits", "e2m1_decode", "e8m0_decode",
    "quantise_blocks", "dequantise_blocks", "pack_nibbles", "unpack_nibbles", "merge_pair_f32",
    "project_key_f32",
    "OracleCache", "BYTES_LATENT", "BYTES_INDEX", "BYTES_PER_ENTRY", "index_scores", "topk_select",
    "hsi_pool", "full_layer", "reindex_layer", "block_summaries", "hisa_layer", "sparse_attention", "gather_rows", "run_decode",
    "run_prefill",
]
