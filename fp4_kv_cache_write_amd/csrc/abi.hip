// extern "C" entry points of libcsa2.so: argument validation, then the launchers.
// The contract of every function is in csa2.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa2.h"
#include "internal.h"

using namespace csa2;

// Workspace of csa2_index_full_noalloc (see scratch_for_current_device below).
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

bool cache_ok(const csa2_cache_t* c) {
  return c && c->lat_codes && c->lat_scales && c->idx_codes && c->idx_scales && c->block_table &&
         c->n_pages > 0 && c->max_pages > 0 && c->ratio >= 0 && c->ratio <= 2;
}

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

// Argument checks shared by csa2_index_full and csa2_index_full_noalloc; on success
// *plan holds the workspace layout the launch will use.
int index_full_check(const csa2_cache_t* cache, int B, const int32_t* ctx_len, int64_t max_ctx,
                     const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                     int cand_block, const int32_t* topk_idx, const int32_t* pool, IndexFullPlan* plan) {
  if (!cache_ok(cache) || B <= 0 || !ctx_len || !q_idx || !w_idx || !topk_idx) return CSA2_EINVAL;
  if (topk < 1 || topk > CSA2_MAX_TOPK || pool_blocks < 0 || max_ctx < 0) return CSA2_EINVAL;
  if (!pow2_in(cand_block, 1, 32)) return CSA2_EINVAL;
  if (pool_blocks > 0 && !pool) return CSA2_EINVAL;
  const int64_t max_nvis = max_ctx >> vis_shift(*cache);
  if (max_nvis > (int64_t)cache->max_pages * CSA2_PAGE) return CSA2_EINVAL;
  *plan = plan_index_full(B, max_nvis, topk, pool_blocks, cand_block);
  if (plan->chunk == 0) return CSA2_EUNSUPPORTED;
  return CSA2_OK;
}

// Workspace of csa2_index_full_noalloc: one array per GPU, resident until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory); it passes the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device and kept.
constexpr size_t kScratchBytes = (size_t)CSA2_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return CSA2_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" {

int csa2_bytes_per_entry(void) {
  return CSA2_LAT_CODE_BYTES + CSA2_LAT_SCALE_BYTES + CSA2_IDX_CODE_BYTES + CSA2_IDX_SCALE_BYTES;
}

const char* csa2_strerror(int code) {
  switch (code) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument";
    case CSA2_EWORKSPACE: return "workspace missing or too small";
    case CSA2_EUNSUPPORTED: return "unsupported request";
    case CSA2_EHIP: return "HIP launch failure";
    case CSA2_ESCRATCH: return "request needs more than the fixed scratch array";
    default: return "unknown error";
  }
}

size_t csa2_workspace_size(int fn, int B, int H, int64_t max_ctx, int topk, int pool_blocks, int C,
                           int ratio) {
  if (B <= 0 || ratio < 0 || ratio > 2) return 0;
  const int vs = ratio == 1 ? 0 : 1;
  switch (fn) {
    case CSA2_FN_INDEX_FULL:
      if (max_ctx < 0 || topk < 1 || topk > CSA2_MAX_TOPK || pool_blocks < 0) return 0;
      // the size does not depend on cand_block; the capacity check here takes the
      // most permissive block size (32), csa2_index_full the caller's
      return plan_index_full(B, max_ctx >> vs, topk, pool_blocks, 32).total;
    case CSA2_FN_REINDEX:
      return reindex_ws(B);
    case CSA2_FN_SPARSE_DECODE:
      if (H <= 0 || topk < 0) return 0;
      return sparse_decode_ws(B, H, topk);
    case CSA2_FN_PREFILL_CHUNK:
      if (H <= 0 || topk < 1 || C <= 0 || max_ctx < 0) return 0;
      return prefill_ws(B, H, max_ctx, topk, C);
    default:
      return 0;
  }
}

int csa2_write_kv(const csa2_cache_t* cache, int B, const int32_t* start_tok, int T_new,
                  const uint16_t* x, const uint16_t* w, const uint16_t* k_idx, int ratio,
                  void* stream) {
  if (!cache_ok(cache) || B <= 0 || !start_tok || !x || !k_idx) return CSA2_EINVAL;
  if (ratio != cache_ratio(*cache)) return CSA2_EINVAL;
  if (ratio == 2 && (!w || T_new <= 0 || (T_new & 1))) return CSA2_EINVAL;
  if (ratio == 1 && T_new <= 0) return CSA2_EINVAL;
  return launch_write_kv(*cache, B, start_tok, T_new, x, w, k_idx, (hipStream_t)stream);
}

int csa2_write_kv_proj(const csa2_cache_t* cache, int B, const int32_t* start_tok, int T_new,
                       const uint16_t* x, const uint16_t* w, const uint16_t* w_proj, int ratio, void* stream) {
  if (!cache_ok(cache) || B <= 0 || !start_tok || !x || !w_proj) return CSA2_EINVAL;
  if (ratio != cache_ratio(*cache)) return CSA2_EINVAL;
  if (ratio == 2 && (!w || T_new <= 0 || (T_new & 1))) return CSA2_EINVAL;
  if (ratio == 1 && T_new <= 0) return CSA2_EINVAL;
  return launch_write_kv_proj(*cache, B, start_tok, T_new, x, w, w_proj, (hipStream_t)stream);
}

int csa2_block_keys(const csa2_cache_t* cache, const csa2_cache_t* blocks, int B, const int32_t* ctx_len,
                    int64_t max_ctx, int cand_block, const int32_t* blk_first, int n_span, int32_t* n_blocks,
                    void* stream) {
  if (!cache_ok(cache) || !cache_ok(blocks) || B <= 0 || !ctx_len || max_ctx < 0) return CSA2_EINVAL;
  if (blocks->ratio != 1 || !pow2_in(cand_block, 1, 32)) return CSA2_EINVAL;
  if (blk_first && n_span < 1) return CSA2_EINVAL;
  return launch_block_keys(*cache, *blocks, B, ctx_len, max_ctx, cand_block, blk_first, n_span, n_blocks,
                           (hipStream_t)stream);
}

int csa2_index_full(const csa2_cache_t* cache, int B, const int32_t* ctx_len, int64_t max_ctx,
                    const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                    int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, size_t ws_bytes,
                    void* stream) {
  IndexFullPlan p{};
  const int rc = index_full_check(cache, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks,
                                  cand_block, topk_idx, pool, &p);
  if (rc != CSA2_OK) return rc;
  if (p.total > 0 && (!ws || ws_bytes < p.total)) return CSA2_EWORKSPACE;
  return launch_index_full(*cache, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks, cand_block,
                           topk_idx, pool, ws, (hipStream_t)stream);
}

int csa2_write_index_full(const csa2_cache_t* cache, int B, const int32_t* start_tok, int T_new,
                          const uint16_t* x, const uint16_t* w, const uint16_t* k_idx, int ratio,
                          const int32_t* ctx_len, int64_t max_ctx, const uint16_t* q_idx, const uint16_t* w_idx,
                          int topk, int pool_blocks, int cand_block, int32_t* topk_idx, int32_t* pool, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!cache_ok(cache) || B <= 0 || !start_tok || !x || !k_idx) return CSA2_EINVAL;
  if (ratio != cache_ratio(*cache)) return CSA2_EINVAL;
  if (ratio == 2 && (!w || T_new <= 0 || (T_new & 1))) return CSA2_EINVAL;
  if (ratio == 1 && T_new <= 0) return CSA2_EINVAL;
  IndexFullPlan p{};
  const int rc = index_full_check(cache, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks,
                                  cand_block, topk_idx, pool, &p);
  if (rc != CSA2_OK) return rc;
  if (p.total > 0 && (!ws || ws_bytes < p.total)) return CSA2_EWORKSPACE;
  return launch_write_index_full(*cache, B, start_tok, T_new, x, w, k_idx, ctx_len, max_ctx, q_idx, w_idx, topk,
                                 pool_blocks, cand_block, topk_idx, pool, ws, (hipStream_t)stream);
}

int csa2_index_full_noalloc(const csa2_cache_t* cache, int B, const int32_t* ctx_len, int64_t max_ctx,
                            const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                            int cand_block, int32_t* topk_idx, int32_t* pool, void* stream) {
  IndexFullPlan p{};
  int rc = index_full_check(cache, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks, cand_block,
                            topk_idx, pool, &p);
  if (rc != CSA2_OK) return rc;
  if (p.total > kScratchBytes) return CSA2_ESCRATCH;
  void* ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc != CSA2_OK) return rc;
  // every workspace byte the kernels read is written earlier in the same launch
  // sequence, so the array's contents from an earlier call need no clearing
  return launch_index_full(*cache, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks, cand_block,
                           topk_idx, pool, ws, (hipStream_t)stream);
}

int csa2_reindex(const csa2_cache_t* cache, int B, const int32_t* ctx_len, const uint16_t* q_idx,
                 const uint16_t* w_idx, const int32_t* pool, int pool_blocks, int cand_block,
                 int topk, int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
  if (!cache_ok(cache) || B <= 0 || !ctx_len || !q_idx || !w_idx || !pool || !topk_idx)
    return CSA2_EINVAL;
  if (ws_bytes > 0 && !ws) return CSA2_EWORKSPACE;
  if (topk < 1 || topk > CSA2_MAX_TOPK || pool_blocks < 1) return CSA2_EINVAL;
  if (!pow2_in(cand_block, 1, 32)) return CSA2_EINVAL;
  if ((int64_t)pool_blocks * cand_block > 16384) return CSA2_EUNSUPPORTED;
  return launch_reindex(*cache, B, ctx_len, q_idx, w_idx, pool, pool_blocks, cand_block, topk,
                        topk_idx, ws, ws ? ws_bytes : 0, (hipStream_t)stream);
}

int csa2_sparse_decode(const csa2_cache_t* cache, int B, int H, const int32_t* ctx_len,
                       const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* swa,
                       int W, float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!cache_ok(cache) || B <= 0 || !ctx_len || !q || !swa || !out) return CSA2_EINVAL;
  if (H <= 0 || (H % 16) != 0 || W < 1 || W > CSA2_MAX_WINDOW) return CSA2_EINVAL;
  if (topk < 0 || topk > CSA2_MAX_TOPK || (topk > 0 && !topk_idx)) return CSA2_EINVAL;
  if (ws_bytes > 0 && !ws) return CSA2_EWORKSPACE;   // the workspace is optional
  return launch_sparse_decode(*cache, B, H, ctx_len, q, topk_idx, topk, swa, W, sm_scale, out, lse,
                              ws, ws_bytes, (hipStream_t)stream);
}

int csa2_prefill_chunk(const csa2_cache_t* cache, int B, int H, const int32_t* prior_len,
                       int64_t max_ctx, int C, const uint16_t* q, const uint16_t* q_idx,
                       const uint16_t* w_idx, const uint16_t* local, int W, int topk,
                       float sm_scale, uint16_t* out, int32_t* topk_idx, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!cache_ok(cache) || B <= 0 || !prior_len || !q || !q_idx || !w_idx || !local || !out)
    return CSA2_EINVAL;
  if (H <= 0 || (H % 16) != 0 || C <= 0 || W < 1 || W > CSA2_MAX_WINDOW) return CSA2_EINVAL;
  if (topk < 1 || topk > CSA2_MAX_TOPK || max_ctx < C) return CSA2_EINVAL;
  if (cache_ratio(*cache) != 2) return CSA2_EUNSUPPORTED;   // the encoder's path
  if (max_ctx / 2 > (int64_t)cache->max_pages * CSA2_PAGE) return CSA2_EINVAL;
  const size_t need = prefill_ws(B, H, max_ctx, topk, C);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_EWORKSPACE;
  return launch_prefill_chunk(*cache, B, H, prior_len, max_ctx, C, q, q_idx, w_idx, local, W, topk,
                              sm_scale, out, topk_idx, ws, (hipStream_t)stream);
}

int csa2_debug_gather(const csa2_cache_t* cache, int B, const int32_t* idx, int n, float* out_lat,
                      float* out_idx, void* stream) {
  if (!cache_ok(cache) || B <= 0 || n < 0 || !idx || (!out_lat && !out_idx)) return CSA2_EINVAL;
  return launch_debug_gather(*cache, B, idx, n, out_lat, out_idx, (hipStream_t)stream);
}

}  // extern "C"
