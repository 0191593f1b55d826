"""The C-ABI library loads, exports what include/csa2.h declares, and rejects bad
host arguments before any launch (CPU only: no compute call reaches the GPU)."""
import ctypes
import os
import re

import pytest

import fp4_kv_cache_write_amd as fk
from fp4_kv_cache_write_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = fk.lib()
    names = _declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(binding.EXPORTS) == set(names)


def test_constants_and_strerror():
    assert fk.bytes_per_entry() == 306
    L = fk.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.csa2_strerror(code) != b"unknown error"
    assert L.csa2_strerror(-99) == b"unknown error"


def test_workspace_sizes_are_consistent():
    a = fk.workspace_size(fk.FN_INDEX_FULL, B=32, max_ctx=65536, topk=512, pool_blocks=512)
    b = fk.workspace_size(fk.FN_INDEX_FULL, B=32, max_ctx=65536, topk=512, pool_blocks=0)
    assert a > 0 and b > 0 and a >= b
    assert fk.workspace_size(fk.FN_INDEX_FULL, B=0, max_ctx=100) == 0
    # a ratio-1 cache has twice the entries for the same tokens: at least as much workspace
    r1 = fk.workspace_size(fk.FN_INDEX_FULL, B=32, max_ctx=65536, topk=512, pool_blocks=512, ratio=1)
    assert r1 >= a
    assert fk.workspace_size(fk.FN_INDEX_FULL, B=32, max_ctx=65536, topk=512, ratio=3) == 0
    assert fk.workspace_size(99, B=1) == 0


def test_index_full_capacity_boundaries():
    # the Full selection merges at most 32,768 candidates (16384-entry chunks x topk) and,
    # with a pool, ranks at most 32,768 block maxima: one entry more is unsupported
    ws = lambda max_ctx, topk, pool_blocks, ratio=2: fk.workspace_size(
        fk.FN_INDEX_FULL, B=1, max_ctx=max_ctx, topk=topk, pool_blocks=pool_blocks, ratio=ratio)
    assert ws(2 * 1048576, 512, 0) > 0 and ws(2 * 1048576 + 2, 512, 0) == 0
    assert ws(1048576, 512, 0, ratio=1) > 0 and ws(1048577, 512, 0, ratio=1) == 0
    assert ws(2 * 16 * 16384, 2048, 0) > 0 and ws(2 * 16 * 16384 + 2, 2048, 0) == 0
    # the pool's block count depends on cand_block: the size query checks with the
    # most permissive (32); the call checks the caller's (EUNSUPPORTED before any launch)
    assert ws(2 * 1048576, 512, 512) > 0 and ws(2 * 1048576 + 2, 512, 512) == 0
    L = fk.lib()
    c, keep = _fake_cache(max_pages=20000)
    p = ctypes.c_void_p(ctypes.addressof(keep))
    call = lambda max_ctx, cand_block: L.csa2_index_full(ctypes.byref(c), 1, p, max_ctx, p, p, 512, 512,
                                                         cand_block, p, p, None, 0, None)
    EWS, EUNS = -2, -3
    assert call(2 * 262144, 8) == EWS and call(2 * 262144 + 2, 8) == EUNS
    assert call(2 * 262144 + 2, 16) == EWS and call(2 * 524288 + 2, 16) == EUNS
    assert call(2 * 32768, 1) == EWS and call(2 * 32768 + 2, 1) == EUNS


def test_index_full_noalloc_limits_return_before_launch():
    # the no-alloc variant checks arguments like csa2_index_full, then refuses a workspace
    # above its fixed array before looking the array up or launching anything
    L = fk.lib()
    c, keep = _fake_cache(max_pages=20000)
    p = ctypes.c_void_p(ctypes.addressof(keep))
    ref = ctypes.byref(c)
    EINVAL, EUNS, ESCRATCH = -1, -3, -5
    limit = 32 << 20
    call = lambda B, max_ctx, pool_blocks, cand_block=8, pool=p: L.csa2_index_full_noalloc(
        ref, B, p, max_ctx, p, p, 512, pool_blocks, cand_block, p, pool, None)
    # batch 128 at 131,072 entries with a 4096-entry pool needs 80 MiB
    assert fk.workspace_size(fk.FN_INDEX_FULL, B=128, max_ctx=262144, topk=512, pool_blocks=512) > limit
    assert call(128, 262144, 512) == ESCRATCH
    # the largest batch that fits is refused one sequence later
    fits = max(B for B in range(1, 200) if fk.workspace_size(
        fk.FN_INDEX_FULL, B=B, max_ctx=262144, topk=512, pool_blocks=512) <= limit)
    assert fits < 128 and call(fits + 1, 262144, 512) == ESCRATCH
    assert call(1, 2 * 262144 + 2, 512) == EUNS          # pool capacity at cand_block 8
    assert call(1, 262144, 512, pool=None) == EINVAL       # pool NULL
    assert call(1, 262144, 0, cand_block=3) == EINVAL
    assert L.csa2_index_full_noalloc(None, 1, p, 128, p, p, 16, 0, 8, p, None, None) == EINVAL


def _fake_cache(max_pages=4, ratio=0):
    # Non-null host addresses: validation must reject the call before anything
    # dereferences them or launches a kernel.
    buf = (ctypes.c_uint8 * 64)()
    addr = ctypes.addressof(buf)
    return binding.CacheT(addr, addr, addr, addr, 4, addr, max_pages, ratio), buf


def test_host_argument_errors_return_before_launch():
    L = fk.lib()
    c, keep = _fake_cache()
    p = ctypes.c_void_p(ctypes.addressof(keep))
    ref = ctypes.byref(c)
    EINVAL, EWS, EUNS = -1, -2, -3
    assert L.csa2_write_kv(None, 1, p, 2, p, p, p, 2, None) == EINVAL
    assert L.csa2_write_kv(ref, 1, p, 3, p, p, p, 2, None) == EINVAL        # odd token count
    assert L.csa2_write_kv(ref, 1, p, 0, p, p, p, 2, None) == EINVAL
    assert L.csa2_write_kv(ref, 1, p, 2, p, p, p, 1, None) == EINVAL       # ratio differs from the cache's
    assert L.csa2_write_kv(ref, 1, None, 2, p, p, p, 2, None) == EINVAL
    assert L.csa2_write_kv(ref, 1, p, 2, p, None, p, 2, None) == EINVAL    # ratio 2 needs w
    assert L.csa2_write_kv_proj(ref, 1, p, 2, p, p, None, 2, None) == EINVAL  # no projection weights
    assert L.csa2_write_kv_proj(ref, 1, p, 3, p, p, p, 2, None) == EINVAL     # odd token count
    assert L.csa2_write_kv_proj(ref, 1, p, 2, p, None, p, 2, None) == EINVAL  # ratio 2 needs w
    assert L.csa2_write_kv_proj(ref, 1, p, 2, p, p, p, 1, None) == EINVAL     # ratio differs from the cache's
    assert L.csa2_write_kv_proj(None, 1, p, 2, p, p, p, 2, None) == EINVAL
    assert L.csa2_block_keys(ref, ref, 1, p, 128, 8, None, 1, None, None) == EINVAL   # block cache not ratio 1
    assert L.csa2_block_keys(ref, None, 1, p, 128, 8, None, 1, None, None) == EINVAL
    assert L.csa2_index_full(ref, 1, p, 128, p, p, 0, 0, 8, p, None, None, 0, None) == EINVAL  # topk 0
    assert L.csa2_index_full(ref, 1, p, 128, p, p, 4096, 0, 8, p, None, None, 0, None) == EINVAL
    assert L.csa2_index_full(ref, 1, p, 128, p, p, 16, 4, 8, p, None, None, 0, None) == EINVAL  # pool NULL
    assert L.csa2_index_full(ref, 1, p, 128, p, p, 16, 0, 3, p, None, None, 0, None) == EINVAL  # block 3
    assert L.csa2_index_full(ref, 1, p, 10 ** 6, p, p, 16, 0, 8, p, None, None, 0, None) == EINVAL  # table too short
    assert L.csa2_index_full(ref, 1, p, 128, p, p, 16, 0, 8, p, None, None, 0, None) == EWS
    assert L.csa2_reindex(ref, 1, p, p, p, p, 0, 8, 16, p, None, 0, None) == EINVAL
    assert L.csa2_reindex(ref, 1, p, p, p, p, 4096, 8, 16, p, None, 0, None) == EUNS
    assert L.csa2_sparse_decode(ref, 1, 12, p, p, p, 16, p, 128, 0.1, p, None, None, 0, None) == EINVAL
    assert L.csa2_sparse_decode(ref, 1, 16, p, p, p, 16, p, 0, 0.1, p, None, None, 0, None) == EINVAL
    assert L.csa2_sparse_decode(ref, 1, 16, p, p, None, 16, p, 128, 0.1, p, None, None, 0, None) == EINVAL
    assert L.csa2_prefill_chunk(ref, 1, 16, p, 128, 0, p, p, p, p, 128, 16, 0.1, p, None, None, 0, None) == EINVAL
    assert L.csa2_debug_gather(ref, 1, p, 4, None, None, None) == EINVAL
    # a ratio-1 (decoder) cache: one entry per token
    c1, keep1 = _fake_cache(ratio=1)
    r1 = ctypes.byref(c1)
    assert L.csa2_write_kv(r1, 1, p, 0, p, None, p, 1, None) == EINVAL      # no tokens
    assert L.csa2_write_kv(r1, 1, p, 3, p, None, p, 2, None) == EINVAL      # ratio differs
    assert L.csa2_index_full(r1, 1, p, 300, p, p, 16, 0, 8, p, None, None, 0, None) == EINVAL  # 300 entries > 256
    assert L.csa2_index_full(r1, 1, p, 200, p, p, 16, 0, 8, p, None, None, 0, None) == EWS
    assert L.csa2_prefill_chunk(r1, 1, 16, p, 128, 64, p, p, p, p, 128, 16, 0.1, p, None, None, 0, None) == EUNS
    bad, keep2 = _fake_cache(ratio=3)
    assert L.csa2_write_kv(ctypes.byref(bad), 1, p, 2, p, p, p, 2, None) == EINVAL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(binding.Csa2Error):
        binding.lib()


def test_schedule_validation_before_capture():
    # invalid schedules are rejected on the host: no stream, capture or launch happens
    L = fk.lib()
    c, keep = _fake_cache()
    p = ctypes.c_void_p(ctypes.addressof(keep))
    EINVAL, EWS = -1, -2

    def layers(*modes, pool=0):
        arr = (binding.LayerT * len(modes))()
        for i, m in enumerate(modes):
            arr[i] = binding.LayerT(binding.LAYER_MODES[m], pool if m == "full" else 0, p, p, p, p, p, None)
        return arr

    ok = layers("full", "reuse", "reindex", "reuse", pool=64)
    assert L.csa2_schedule_workspace_size(2, 16, 4096, 64, 4, ok, 2) > 0
    assert L.csa2_schedule_workspace_size(2, 16, 4096, 64, 1, layers("reuse"), 2) == 0        # no selection yet
    assert L.csa2_schedule_workspace_size(2, 16, 4096, 64, 2, layers("full", "reindex"), 2) == 0  # no pool
    assert L.csa2_schedule_workspace_size(2, 12, 4096, 64, 4, ok, 2) == 0                      # H % 16
    assert L.csa2_schedule_workspace_size(2, 16, 4096, 64, 4, ok, 3) == 0                      # ratio
    out = ctypes.c_void_p()
    ref = ctypes.byref(c)
    args = (ref, 2, 16, p, 400, 64, 8, 128, 0.1, None, 0, None, None, None)   # 200 entries fit 4 pages
    assert L.csa2_schedule_create(*args, 4, ok, p, 0, ctypes.byref(out)) == EWS and not out.value
    assert L.csa2_schedule_create(*args, 1, layers("reuse"), p, 1 << 30, ctypes.byref(out)) == EINVAL
    assert L.csa2_schedule_create(*args, 4, ok, p, 1 << 30, None) == EINVAL
    assert L.csa2_schedule_launch(None, None) == EINVAL
    L.csa2_schedule_destroy(None)


def test_write_index_full_rejects_what_either_call_rejects():
    L = fk.lib()
    c, keep = _fake_cache()
    p = ctypes.c_void_p(ctypes.addressof(keep))
    ref = ctypes.byref(c)
    EINVAL, EWS, EUNS = -1, -2, -3

    def call(T_new=2, x=p, w=p, k=p, ratio=2, ctx=p, max_ctx=128, q=p, topk=16, pool_blocks=0, cand_block=8,
             pool=None, ws=None, ws_bytes=0, cache=ref, start=p):
        return L.csa2_write_index_full(cache, 1, start, T_new, x, w, k, ratio, ctx, max_ctx, q, p, topk,
                                       pool_blocks, cand_block, p, pool, ws, ws_bytes, None)

    assert call() == EWS                      # valid arguments, no workspace: nothing launched
    assert call(cache=None) == EINVAL
    assert call(start=None) == EINVAL
    assert call(T_new=3) == EINVAL            # odd token count at ratio 2
    assert call(T_new=0) == EINVAL
    assert call(ratio=1) == EINVAL            # ratio differs from the cache's
    assert call(w=None) == EINVAL             # ratio 2 needs w
    assert call(k=None) == EINVAL
    assert call(q=None) == EINVAL
    assert call(ctx=None) == EINVAL
    assert call(topk=0) == EINVAL
    assert call(cand_block=3) == EINVAL
    assert call(pool_blocks=4) == EINVAL      # pool NULL
    assert call(max_ctx=2 * 4 * 64 + 2) == EINVAL   # beyond the table's pages
