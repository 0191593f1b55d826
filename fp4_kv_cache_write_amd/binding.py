"""ctypes binding of libcsa2.so — argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the path
runs in the library's HIP kernels.  There is no fallback: a missing library or a
failed call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

# CSA2_LIB may name another build of the same library (same ABI).
_LIB_PATH = os.environ.get("CSA2_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

D_LATENT, D_INDEX, H_INDEX, PAGE = 512, 64, 4, 64
FN_INDEX_FULL, FN_REINDEX, FN_SPARSE_DECODE, FN_PREFILL_CHUNK = 1, 2, 3, 4

EXPORTS = ("csa2_bytes_per_entry", "csa2_strerror", "csa2_workspace_size", "csa2_write_kv", "csa2_write_kv_proj", "csa2_block_keys",
           "csa2_index_full", "csa2_write_index_full", "csa2_index_full_noalloc", "csa2_reindex", "csa2_sparse_decode", "csa2_prefill_chunk",
           "csa2_debug_gather", "csa2_schedule_workspace_size", "csa2_schedule_create",
           "csa2_schedule_launch", "csa2_schedule_destroy")
LAYER_MODES = {"full": 0, "reindex": 1, "reuse": 2}


class Csa2Error(RuntimeError):
    pass


class LayerT(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("pool_blocks", ctypes.c_int32), ("q", ctypes.c_void_p),
                ("q_idx", ctypes.c_void_p), ("w_idx", ctypes.c_void_p), ("swa", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class CacheT(ctypes.Structure):
    _fields_ = [("lat_codes", ctypes.c_void_p), ("lat_scales", ctypes.c_void_p),
                ("idx_codes", ctypes.c_void_p), ("idx_scales", ctypes.c_void_p),
                ("n_pages", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("max_pages", ctypes.c_int32), ("ratio", ctypes.c_int32)]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise Csa2Error(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        P, I, I64, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        C = ctypes.POINTER(CacheT)
        L.csa2_bytes_per_entry.restype = I
        L.csa2_bytes_per_entry.argtypes = []
        L.csa2_strerror.restype = ctypes.c_char_p
        L.csa2_strerror.argtypes = [I]
        L.csa2_workspace_size.restype = SZ
        L.csa2_workspace_size.argtypes = [I, I, I, I64, I, I, I, I]
        L.csa2_write_kv.restype = I
        L.csa2_write_kv.argtypes = [C, I, P, I, P, P, P, I, P]
        L.csa2_write_kv_proj.restype = I
        L.csa2_write_kv_proj.argtypes = [C, I, P, I, P, P, P, I, P]
        L.csa2_block_keys.restype = I
        L.csa2_block_keys.argtypes = [C, C, I, P, I64, I, P, I, P, P]
        L.csa2_index_full.restype = I
        L.csa2_index_full.argtypes = [C, I, P, I64, P, P, I, I, I, P, P, P, SZ, P]
        L.csa2_write_index_full.restype = I
        L.csa2_write_index_full.argtypes = [C, I, P, I, P, P, P, I, P, I64, P, P, I, I, I, P, P, P, SZ, P]
        L.csa2_index_full_noalloc.restype = I
        L.csa2_index_full_noalloc.argtypes = [C, I, P, I64, P, P, I, I, I, P, P, P]
        L.csa2_reindex.restype = I
        L.csa2_reindex.argtypes = [C, I, P, P, P, P, I, I, I, P, P, SZ, P]
        L.csa2_sparse_decode.restype = I
        L.csa2_sparse_decode.argtypes = [C, I, I, P, P, P, I, P, I, F, P, P, P, SZ, P]
        L.csa2_prefill_chunk.restype = I
        L.csa2_prefill_chunk.argtypes = [C, I, I, P, I64, I, P, P, P, P, I, I, F, P, P, P, SZ, P]
        L.csa2_debug_gather.restype = I
        L.csa2_debug_gather.argtypes = [C, I, P, I, P, P, P]
        LP = ctypes.POINTER(LayerT)
        L.csa2_schedule_workspace_size.restype = SZ
        L.csa2_schedule_workspace_size.argtypes = [I, I, I64, I, I, LP, I]
        L.csa2_schedule_create.restype = I
        L.csa2_schedule_create.argtypes = [C, I, I, P, I64, I, I, I, F, P, I, P, P, P, I, LP, P, SZ,
                                           ctypes.POINTER(P)]
        L.csa2_schedule_launch.restype = I
        L.csa2_schedule_launch.argtypes = [P, P]
        L.csa2_schedule_destroy.restype = None
        L.csa2_schedule_destroy.argtypes = [P]
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise Csa2Error(f"{what}: {lib().csa2_strerror(rc).decode()} ({rc})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str, shape=None) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _bf16(t: torch.Tensor, name: str, shape=None) -> None:
    _need(t, torch.bfloat16, name, shape)


class PagedCache:
    """Device byte arrays of the paged FP4 cache plus its block table (see csa2.h).

    ratio: tokens per entry, 2 (encoder: token pairs merged) or 1 (decoder: one entry
    per token)."""

    def __init__(self, lat_codes, lat_scales, idx_codes, idx_scales, block_table, ratio: int = 2):
        if ratio not in (1, 2):
            raise Csa2Error(f"ratio must be 1 or 2, got {ratio}")
        self.ratio = ratio
        self.lat_codes, self.lat_scales = lat_codes, lat_scales
        self.idx_codes, self.idx_scales = idx_codes, idx_scales
        self.block_table = block_table
        for name in ("lat_codes", "lat_scales", "idx_codes", "idx_scales"):
            _need(getattr(self, name), torch.uint8, name)
        _need(block_table, torch.int32, "block_table")
        self.n_pages = lat_codes.shape[0]
        self.max_pages = block_table.shape[1]
        self._struct = CacheT(lat_codes.data_ptr(), lat_scales.data_ptr(), idx_codes.data_ptr(),
                              idx_scales.data_ptr(), self.n_pages, block_table.data_ptr(),
                              self.max_pages, ratio)

    @classmethod
    def allocate(cls, n_pages: int, block_table: torch.Tensor, device="cuda", fill: int = 0, ratio: int = 2):
        mk = lambda *s: torch.full(s, fill, dtype=torch.uint8, device=device)
        return cls(mk(n_pages, PAGE, D_LATENT // 2), mk(n_pages, PAGE, D_LATENT // 32),
                   mk(n_pages, PAGE, D_INDEX // 2), mk(n_pages, PAGE, D_INDEX // 32),
                   block_table.to(device=device, dtype=torch.int32).contiguous(), ratio)

    def clone(self) -> "PagedCache":
        return PagedCache(self.lat_codes.clone(), self.lat_scales.clone(), self.idx_codes.clone(),
                          self.idx_scales.clone(), self.block_table.clone(), self.ratio)

    def rows(self, b0: int, b1: int) -> "PagedCache":
        """The same cache with the block-table rows of sequences b0 .. b1-1 only."""
        return PagedCache(self.lat_codes, self.lat_scales, self.idx_codes, self.idx_scales,
                          self.block_table[b0:b1].contiguous(), self.ratio)

    @property
    def ref(self):
        return ctypes.byref(self._struct)

    @property
    def B(self) -> int:
        return self.block_table.shape[0]


def bytes_per_entry() -> int:
    return lib().csa2_bytes_per_entry()


def workspace_size(fn: int, B: int, H: int = 0, max_ctx: int = 0, topk: int = 512,
                   pool_blocks: int = 0, C: int = 0, ratio: int = 2) -> int:
    return lib().csa2_workspace_size(fn, B, H, max_ctx, topk, pool_blocks, C, ratio)


def workspace(fn: int, device="cuda", **kw) -> Optional[torch.Tensor]:
    n = workspace_size(fn, **kw)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device) if n > 0 else None


def write_kv(cache: PagedCache, start_tok: torch.Tensor, x: torch.Tensor, w: Optional[torch.Tensor],
             k_idx: torch.Tensor, ratio: Optional[int] = None, stream=None) -> None:
    """Write tokens start_tok .. start_tok+T-1 of every sequence.  ratio defaults to the
    cache's; at ratio 1 w is unused (None) and k_idx has one key per token."""
    ratio = cache.ratio if ratio is None else ratio
    B, T = x.shape[0], x.shape[1]
    _bf16(x, "x", (B, T, D_LATENT))
    if ratio == 2 or w is not None:
        _bf16(w, "w", (B, T, D_LATENT))
    _bf16(k_idx, "k_idx", (B, T // ratio, D_INDEX))
    _need(start_tok, torch.int32, "start_tok", (B,))
    _check(lib().csa2_write_kv(cache.ref, B, _ptr(start_tok), T, _ptr(x), _ptr(w), _ptr(k_idx), ratio,
                               _stream(stream)), "csa2_write_kv")



def write_kv_proj(cache: PagedCache, start_tok: torch.Tensor, x: torch.Tensor, w: Optional[torch.Tensor],
                  w_proj: torch.Tensor, ratio: Optional[int] = None, stream=None) -> None:
    """Write tokens start_tok .. start_tok+T-1 of every sequence with each entry's indexer
    key projected from the entry by w_proj [64][512] (bf16) inside the kernel."""
    ratio = cache.ratio if ratio is None else ratio
    B, T = x.shape[0], x.shape[1]
    _bf16(x, "x", (B, T, D_LATENT))
    if ratio == 2 or w is not None:
        _bf16(w, "w", (B, T, D_LATENT))
    _bf16(w_proj, "w_proj", (D_INDEX, D_LATENT))
    _need(start_tok, torch.int32, "start_tok", (B,))
    _check(lib().csa2_write_kv_proj(cache.ref, B, _ptr(start_tok), T, _ptr(x), _ptr(w), _ptr(w_proj), ratio,
                                    _stream(stream)), "csa2_write_kv_proj")


def block_keys(cache: PagedCache, blocks: PagedCache, ctx_len: torch.Tensor, max_ctx: int, cand_block: int = 8,
               blk_first: Optional[torch.Tensor] = None, n_span: int = 1, n_blocks: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """HISA block summaries of cache's indexer keys into `blocks` (a ratio-1 cache whose
    slot k holds block k); all blocks, or per sequence blk_first[b] .. +n_span-1.
    Returns the per-sequence block counts (the context to index `blocks` with)."""
    B = ctx_len.shape[0]
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    if blk_first is not None:
        _need(blk_first, torch.int32, "blk_first", (B,))
    if n_blocks is None:
        n_blocks = torch.empty((B,), dtype=torch.int32, device=ctx_len.device)
    _check(lib().csa2_block_keys(cache.ref, blocks.ref, B, _ptr(ctx_len), max_ctx, cand_block, _ptr(blk_first),
                                 n_span, _ptr(n_blocks), _stream(stream)), "csa2_block_keys")
    return n_blocks


def index_hisa(cache: PagedCache, blocks: PagedCache, n_blocks: torch.Tensor, max_blocks: int, ctx_len: torch.Tensor,
               q_idx: torch.Tensor, w_idx: torch.Tensor, keep_blocks: int, topk: int = 512, cand_block: int = 8,
               ws_blocks: Optional[torch.Tensor] = None, ws_reindex: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """HISA selection: the keep_blocks best block summaries (csa2_index_full on `blocks`),
    then the top-K of their entries (csa2_reindex on `cache`).  Returns (top-K, pool)."""
    pool, _ = index_full(blocks, n_blocks, max_blocks, q_idx, w_idx, topk=keep_blocks, pool_blocks=0,
                         cand_block=cand_block, ws=ws_blocks, stream=stream)
    tk = reindex(cache, ctx_len, q_idx, w_idx, pool, topk=topk, cand_block=cand_block, ws=ws_reindex, stream=stream)
    return tk, pool

def index_full(cache: PagedCache, ctx_len: torch.Tensor, max_ctx: int, q_idx: torch.Tensor,
               w_idx: torch.Tensor, topk: int = 512, pool_blocks: int = 0, cand_block: int = 8,
               ws: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
               pool: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    B = ctx_len.shape[0]
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    _bf16(q_idx, "q_idx", (B, H_INDEX, D_INDEX))
    _bf16(w_idx, "w_idx", (B, H_INDEX))
    dev = q_idx.device
    if topk_idx is None:
        topk_idx = torch.empty((B, topk), dtype=torch.int32, device=dev)
    if pool_blocks > 0 and pool is None:
        pool = torch.empty((B, pool_blocks), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(FN_INDEX_FULL, device=dev, B=B, max_ctx=max_ctx, topk=topk, pool_blocks=pool_blocks,
                       ratio=cache.ratio)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().csa2_index_full(cache.ref, B, _ptr(ctx_len), max_ctx, _ptr(q_idx), _ptr(w_idx), topk,
                                 pool_blocks, cand_block, _ptr(topk_idx), _ptr(pool), _ptr(ws), wsb,
                                 _stream(stream)), "csa2_index_full")
    return topk_idx, pool


def write_index_full(cache: PagedCache, start_tok: torch.Tensor, x: torch.Tensor, w: Optional[torch.Tensor],
                     k_idx: torch.Tensor, ctx_len: torch.Tensor, max_ctx: int, q_idx: torch.Tensor,
                     w_idx: torch.Tensor, topk: int = 512, pool_blocks: int = 0, cand_block: int = 8,
                     ws: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                     pool: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """csa2_write_index_full: write_kv(cache, start_tok, x, w, k_idx) then index_full(...),
    in one launch sequence with the same results."""
    ratio = cache.ratio
    B, T = x.shape[0], x.shape[1]
    _bf16(x, "x", (B, T, D_LATENT))
    if ratio == 2 or w is not None:
        _bf16(w, "w", (B, T, D_LATENT))
    _bf16(k_idx, "k_idx", (B, T // ratio, D_INDEX))
    _need(start_tok, torch.int32, "start_tok", (B,))
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    _bf16(q_idx, "q_idx", (B, H_INDEX, D_INDEX))
    _bf16(w_idx, "w_idx", (B, H_INDEX))
    dev = q_idx.device
    if topk_idx is None:
        topk_idx = torch.empty((B, topk), dtype=torch.int32, device=dev)
    if pool_blocks > 0 and pool is None:
        pool = torch.empty((B, pool_blocks), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(FN_INDEX_FULL, device=dev, B=B, max_ctx=max_ctx, topk=topk, pool_blocks=pool_blocks,
                       ratio=ratio)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().csa2_write_index_full(cache.ref, B, _ptr(start_tok), T, _ptr(x), _ptr(w), _ptr(k_idx), ratio,
                                       _ptr(ctx_len), max_ctx, _ptr(q_idx), _ptr(w_idx), topk, pool_blocks,
                                       cand_block, _ptr(topk_idx), _ptr(pool), _ptr(ws), wsb, _stream(stream)),
           "csa2_write_index_full")
    return topk_idx, pool


def index_full_noalloc(cache: PagedCache, ctx_len: torch.Tensor, max_ctx: int, q_idx: torch.Tensor,
                       w_idx: torch.Tensor, topk_idx: torch.Tensor, pool: Optional[torch.Tensor] = None,
                       topk: int = 512, pool_blocks: int = 0, cand_block: int = 8, stream=None) -> None:
    """csa2_index_full_noalloc: outputs are the caller's; the workspace is the library's
    fixed per-GPU array, so nothing is allocated on this path."""
    B = ctx_len.shape[0]
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    _bf16(q_idx, "q_idx", (B, H_INDEX, D_INDEX))
    _bf16(w_idx, "w_idx", (B, H_INDEX))
    _need(topk_idx, torch.int32, "topk_idx", (B, topk))
    if pool_blocks > 0:
        if pool is None:
            raise ValueError("pool is required when pool_blocks > 0")
        _need(pool, torch.int32, "pool", (B, pool_blocks))
    _check(lib().csa2_index_full_noalloc(cache.ref, B, _ptr(ctx_len), max_ctx, _ptr(q_idx), _ptr(w_idx),
                                         topk, pool_blocks, cand_block, _ptr(topk_idx), _ptr(pool),
                                         _stream(stream)), "csa2_index_full_noalloc")


def reindex(cache: PagedCache, ctx_len: torch.Tensor, q_idx: torch.Tensor, w_idx: torch.Tensor,
            pool: torch.Tensor, topk: int = 512, cand_block: int = 8,
            topk_idx: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
            split: bool = True, stream=None) -> torch.Tensor:
    B = ctx_len.shape[0]
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    _bf16(q_idx, "q_idx", (B, H_INDEX, D_INDEX))
    _bf16(w_idx, "w_idx", (B, H_INDEX))
    _need(pool, torch.int32, "pool")
    if topk_idx is None:
        topk_idx = torch.empty((B, topk), dtype=torch.int32, device=q_idx.device)
    if ws is None and split:
        ws = workspace(FN_REINDEX, device=q_idx.device, B=B, topk=topk, pool_blocks=pool.shape[1],
                       ratio=cache.ratio)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().csa2_reindex(cache.ref, B, _ptr(ctx_len), _ptr(q_idx), _ptr(w_idx), _ptr(pool),
                              pool.shape[1], cand_block, topk, _ptr(topk_idx), _ptr(ws), wsb, _stream(stream)),
           "csa2_reindex")
    return topk_idx


def sparse_decode(cache: PagedCache, ctx_len: torch.Tensor, q: torch.Tensor, topk_idx: torch.Tensor,
                  swa: torch.Tensor, sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                  ws: Optional[torch.Tensor] = None, stream=None):
    B, H = q.shape[0], q.shape[1]
    W = swa.shape[1]
    _need(ctx_len, torch.int32, "ctx_len", (B,))
    _bf16(q, "q", (B, H, D_LATENT))
    _bf16(swa, "swa", (B, W, D_LATENT))
    _need(topk_idx, torch.int32, "topk_idx")
    topk = topk_idx.shape[1]
    if sm_scale is None:
        sm_scale = D_LATENT ** -0.5
    if out is None:
        out = torch.empty((B, H, D_LATENT), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if ws is None:   # split partials: every byte used is written first, no clearing needed
        n = workspace_size(FN_SPARSE_DECODE, B=B, H=H, topk=topk)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    wsb = ws.numel() if ws is not None else 0
    _check(lib().csa2_sparse_decode(cache.ref, B, H, _ptr(ctx_len), _ptr(q), _ptr(topk_idx), topk,
                                    _ptr(swa), W, sm_scale, _ptr(out), _ptr(lse), _ptr(ws), wsb,
                                    _stream(stream)), "csa2_sparse_decode")
    return out, lse


def prefill_chunk(cache: PagedCache, prior_len: torch.Tensor, max_ctx: int, q: torch.Tensor,
                  q_idx: torch.Tensor, w_idx: torch.Tensor, local: torch.Tensor, topk: int = 512,
                  sm_scale: Optional[float] = None, want_topk: bool = True,
                  out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                  topk_idx: Optional[torch.Tensor] = None, stream=None):
    B, C, H = q.shape[0], q.shape[1], q.shape[2]
    W = local.shape[1] - C + 1
    _need(prior_len, torch.int32, "prior_len", (B,))
    _bf16(q, "q", (B, C, H, D_LATENT))
    _bf16(q_idx, "q_idx", (B, C, H_INDEX, D_INDEX))
    _bf16(w_idx, "w_idx", (B, C, H_INDEX))
    _bf16(local, "local", (B, W - 1 + C, D_LATENT))
    if sm_scale is None:
        sm_scale = D_LATENT ** -0.5
    if out is None:
        out = torch.empty((B, C, H, D_LATENT), dtype=torch.bfloat16, device=q.device)
    if topk_idx is not None:
        _need(topk_idx, torch.int32, "topk_idx", (B, C, topk))
        tk = topk_idx
    else:
        tk = torch.empty((B, C, topk), dtype=torch.int32, device=q.device) if want_topk else None
    if ws is None:
        ws = workspace(FN_PREFILL_CHUNK, device=q.device, B=B, H=H, max_ctx=max_ctx, topk=topk, C=C)
    wsb = ws.numel() if ws is not None else 0
    _check(lib().csa2_prefill_chunk(cache.ref, B, H, _ptr(prior_len), max_ctx, C, _ptr(q), _ptr(q_idx),
                                    _ptr(w_idx), _ptr(local), W, topk, sm_scale, _ptr(out), _ptr(tk),
                                    _ptr(ws), wsb, _stream(stream)), "csa2_prefill_chunk")
    return out, tk


def debug_gather(cache: PagedCache, idx: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    B, n = idx.shape
    _need(idx, torch.int32, "idx")
    lat = torch.empty((B, n, D_LATENT), dtype=torch.float32, device=idx.device)
    key = torch.empty((B, n, D_INDEX), dtype=torch.float32, device=idx.device)
    _check(lib().csa2_debug_gather(cache.ref, B, _ptr(idx), n, _ptr(lat), _ptr(key), _stream(stream)),
           "csa2_debug_gather")
    return lat, key


class Schedule:
    """One decode step of a layer schedule captured into a HIP graph (csa2_schedule_*).

    layers: list of dicts with mode ("full" | "reindex" | "reuse"), pool_blocks (Full),
    q, q_idx, w_idx (Full, Reindex), swa, out and optional lse tensors.  write: optional
    dict (start, x, w, k) of the step's write.  The tensors are kept alive with the
    schedule; their contents are read when launch() runs the graph.
    """

    def __init__(self, cache: PagedCache, ctx_len: torch.Tensor, max_ctx: int, layers, W: int,
                 topk: int = 512, cand_block: int = 8, sm_scale: Optional[float] = None, write=None,
                 ws: Optional[torch.Tensor] = None):
        B = ctx_len.shape[0]
        _need(ctx_len, torch.int32, "ctx_len", (B,))
        H = layers[0]["q"].shape[1]
        if sm_scale is None:
            sm_scale = D_LATENT ** -0.5
        arr = (LayerT * len(layers))()
        keep = [cache, ctx_len]
        for i, L in enumerate(layers):
            _bf16(L["q"], "q", (B, H, D_LATENT))
            _bf16(L["swa"], "swa", (B, W, D_LATENT))
            _bf16(L["out"], "out", (B, H, D_LATENT))
            if L["mode"] != "reuse":
                _bf16(L["q_idx"], "q_idx", (B, H_INDEX, D_INDEX))
                _bf16(L["w_idx"], "w_idx", (B, H_INDEX))
            arr[i] = LayerT(LAYER_MODES[L["mode"]], L.get("pool_blocks", 0), _ptr(L["q"]), _ptr(L.get("q_idx")),
                            _ptr(L.get("w_idx")), _ptr(L["swa"]), _ptr(L["out"]), _ptr(L.get("lse")))
            keep += [v for v in L.values() if isinstance(v, torch.Tensor)]
        n = lib().csa2_schedule_workspace_size(B, H, max_ctx, topk, len(layers), arr, cache.ratio)
        if n == 0:
            raise Csa2Error("csa2_schedule_workspace_size: invalid schedule")
        if ws is None:
            ws = torch.empty(n, dtype=torch.uint8, device=ctx_len.device)
        keep.append(ws)
        wr = write or {}
        x, w, k, start = wr.get("x"), wr.get("w"), wr.get("k"), wr.get("start")
        T = x.shape[1] if x is not None else 0
        keep += [t for t in (x, w, k, start) if t is not None]
        handle = ctypes.c_void_p()
        _check(lib().csa2_schedule_create(cache.ref, B, H, _ptr(ctx_len), max_ctx, topk, cand_block, W, sm_scale,
                                          _ptr(start), T, _ptr(x), _ptr(w), _ptr(k), len(layers), arr, _ptr(ws),
                                          ws.numel(), ctypes.byref(handle)), "csa2_schedule_create")
        self._handle = handle
        self._keep = keep

    def launch(self, stream=None) -> None:
        _check(lib().csa2_schedule_launch(self._handle, _stream(stream)), "csa2_schedule_launch")

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            lib().csa2_schedule_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
