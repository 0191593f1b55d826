"""CSA2 compressed-KV sparse decode for MI355X (gfx950).

The compute path is libcsa2.so (hand-written HIP kernels behind a C ABI,
include/csa2.h); this package is its ctypes binding.  There is no CPU or
PyTorch fallback.
"""
from . import binding
from .binding import (Csa2Error, PagedCache, Schedule, block_keys, bytes_per_entry, debug_gather, index_full,
                      index_full_noalloc,
                      index_hisa, lib,
                      prefill_chunk, reindex, sparse_decode, workspace, workspace_size, write_index_full, write_kv,
                      write_kv_proj, FN_INDEX_FULL, FN_REINDEX, FN_SPARSE_DECODE, FN_PREFILL_CHUNK)

__all__ = ["binding", "Csa2Error", "PagedCache", "Schedule", "block_keys", "bytes_per_entry", "debug_gather",
           "index_full", "index_full_noalloc", "index_hisa", "lib",
           "prefill_chunk", "reindex", "sparse_decode", "workspace", "workspace_size", "write_index_full", "write_kv",
           "write_kv_proj", "FN_INDEX_FULL", "FN_REINDEX", "FN_SPARSE_DECODE", "FN_PREFILL_CHUNK"]
