// Layer-schedule runner: one decode step of a CSA2 layer schedule -- the step's write,
// then for every layer its selection (Full or Reindex, or none for Reuse) and its
// attention -- captured once into a HIP graph and replayed with one launch.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §2.3.2 (Full, Reindex and
// Reuse modes share one cache; Reuse takes the latest selection) and §2.3.3 (an
// encoder block is one Full layer and five Reuse layers; the decoder runs a Full
// block with three Reuse layers, then four blocks of one Reindex and three Reuse
// layers).
//
// Host code only.  The calls are the library's own launchers, issued in layer order
// on a private capture stream, on the same buffers the separate calls would use; a
// step whose first layer is Full runs its write inside that layer's scan (the launch
// of csa2_write_index_full), so the graph's results are those of the separate calls.
// Intermediates (the current selection, the pool, the workspaces of the index,
// Reindex and attention calls) live in one caller workspace; the graph and its
// executable are the only allocations (host-side objects of the HIP runtime).
#include <hip/hip_runtime.h>

#include <new>

#include "csa2.h"
#include "internal.h"

using namespace csa2;

struct csa2_schedule {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct SchedLayout {
  size_t off_topk, off_pool, off_full, off_re, off_att, total;
  int pool_blocks;   // largest pool quota of the schedule's Full layers
};

// Checks the schedule's shape and lays out its workspace; returns CSA2_OK or a code.
int plan_schedule(int B, int H, int64_t max_ctx, int topk, int n_layers, const csa2_layer_t* layers, int ratio,
                  SchedLayout* out) {
  if (B <= 0 || H <= 0 || (H % 16) != 0 || topk < 1 || topk > CSA2_MAX_TOPK || max_ctx < 0) return CSA2_EINVAL;
  if (n_layers < 1 || !layers) return CSA2_EINVAL;
  int pool_blocks = 0;
  bool have_sel = false, have_pool = false;
  for (int l = 0; l < n_layers; ++l) {
    const csa2_layer_t& L = layers[l];
    switch (L.mode) {
      case CSA2_LAYER_FULL:
        if (L.pool_blocks < 0) return CSA2_EINVAL;
        if (L.pool_blocks > pool_blocks) pool_blocks = L.pool_blocks;
        have_sel = true;
        have_pool = L.pool_blocks > 0;
        break;
      case CSA2_LAYER_REINDEX:
        if (!have_pool) return CSA2_EINVAL;   // needs an earlier Full layer's pool
        have_sel = true;
        break;
      case CSA2_LAYER_REUSE:
        if (!have_sel) return CSA2_EINVAL;    // needs an earlier selection
        break;
      default:
        return CSA2_EINVAL;
    }
  }
  const int vs = ratio == 1 ? 0 : 1;
  const IndexFullPlan ip = plan_index_full(B, max_ctx >> vs, topk, pool_blocks, 8);
  if (ip.chunk == 0) return CSA2_EUNSUPPORTED;
  SchedLayout s{};
  s.pool_blocks = pool_blocks;
  size_t off = 0;
  s.off_topk = off;
  off = align256(off + (size_t)B * topk * 4);
  s.off_pool = off;
  off = align256(off + (size_t)B * (pool_blocks > 0 ? pool_blocks : 1) * 4);
  s.off_full = off;
  off = align256(off + ip.total);
  s.off_re = off;
  off = align256(off + reindex_ws(B));
  s.off_att = off;
  off = align256(off + sparse_decode_ws(B, H, topk));
  s.total = off;
  *out = s;
  return CSA2_OK;
}

}  // namespace

extern "C" {

size_t csa2_schedule_workspace_size(int B, int H, int64_t max_ctx, int topk, int n_layers,
                                    const csa2_layer_t* layers, int ratio) {
  if (ratio < 0 || ratio > 2) return 0;
  SchedLayout s;
  return plan_schedule(B, H, max_ctx, topk, n_layers, layers, ratio == 1 ? 1 : 2, &s) == CSA2_OK ? s.total : 0;
}

int csa2_schedule_create(const csa2_cache_t* cache, int B, int H, const int32_t* ctx_len, int64_t max_ctx,
                         int topk, int cand_block, int W, float sm_scale, const int32_t* start_tok, int T_new,
                         const uint16_t* x, const uint16_t* w, const uint16_t* k_idx, int n_layers,
                         const csa2_layer_t* layers, void* ws, size_t ws_bytes, csa2_schedule_t** out) {
  if (!out) return CSA2_EINVAL;
  *out = nullptr;
  if (!cache || !ctx_len || W < 1 || W > CSA2_MAX_WINDOW) return CSA2_EINVAL;
  if (!(cand_block >= 1 && cand_block <= 32 && (cand_block & (cand_block - 1)) == 0)) return CSA2_EINVAL;
  if (cache->ratio < 0 || cache->ratio > 2 || cache->n_pages <= 0 || cache->max_pages <= 0) return CSA2_EINVAL;
  const int ratio = cache_ratio(*cache);
  if ((max_ctx >> vis_shift(*cache)) > (int64_t)cache->max_pages * CSA2_PAGE) return CSA2_EINVAL;
  SchedLayout s;
  const int rc = plan_schedule(B, H, max_ctx, topk, n_layers, layers, ratio, &s);
  if (rc != CSA2_OK) return rc;
  if (!ws || ws_bytes < s.total) return CSA2_EWORKSPACE;
  for (int l = 0; l < n_layers; ++l) {
    const csa2_layer_t& L = layers[l];
    if (!L.q || !L.swa || !L.out) return CSA2_EINVAL;
    if (L.mode != CSA2_LAYER_REUSE && (!L.q_idx || !L.w_idx)) return CSA2_EINVAL;
    if (L.mode == CSA2_LAYER_REINDEX && (int64_t)s.pool_blocks * cand_block > 16384) return CSA2_EUNSUPPORTED;
  }
  if (x) {   // the step's write
    if (!start_tok || !k_idx || T_new <= 0) return CSA2_EINVAL;
    if (ratio == 2 && (!w || (T_new & 1))) return CSA2_EINVAL;
  }
  if (!index_kernels_ready() || !attention_kernels_ready()) return CSA2_EHIP;

  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* topk_idx = reinterpret_cast<int32_t*>(base + s.off_topk);
  int32_t* pool = reinterpret_cast<int32_t*>(base + s.off_pool);
  void* ws_full = base + s.off_full;
  void* ws_re = base + s.off_re;
  void* ws_att = base + s.off_att;
  const size_t re_bytes = s.off_att - s.off_re;
  const size_t att_bytes = s.total - s.off_att;

  hipStream_t st = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return CSA2_EHIP;
  if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(st);
    return CSA2_EHIP;
  }
  int err = CSA2_OK;
  const bool fused_write = x && layers[0].mode == CSA2_LAYER_FULL;
  if (x && !fused_write) err = launch_write_kv(*cache, B, start_tok, T_new, x, w, k_idx, st);
  int cur_pool_blocks = 0;
  for (int l = 0; l < n_layers && err == CSA2_OK; ++l) {
    const csa2_layer_t& L = layers[l];
    if (L.mode == CSA2_LAYER_FULL && l == 0 && fused_write) {
      cur_pool_blocks = L.pool_blocks;
      err = launch_write_index_full(*cache, B, start_tok, T_new, x, w, k_idx, ctx_len, max_ctx, L.q_idx, L.w_idx,
                                    topk, L.pool_blocks, cand_block, topk_idx, L.pool_blocks > 0 ? pool : nullptr,
                                    ws_full, st);
    } else if (L.mode == CSA2_LAYER_FULL) {
      cur_pool_blocks = L.pool_blocks;
      err = launch_index_full(*cache, B, ctx_len, max_ctx, L.q_idx, L.w_idx, topk, L.pool_blocks, cand_block,
                              topk_idx, L.pool_blocks > 0 ? pool : nullptr, ws_full, st);
    } else if (L.mode == CSA2_LAYER_REINDEX) {
      err = launch_reindex(*cache, B, ctx_len, L.q_idx, L.w_idx, pool, cur_pool_blocks, cand_block, topk, topk_idx,
                           ws_re, re_bytes, st);
    }
    if (err == CSA2_OK)
      err = launch_sparse_decode(*cache, B, H, ctx_len, L.q, topk_idx, topk, L.swa, W, sm_scale, L.out, L.lse,
                                 ws_att, att_bytes, st);
  }
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(st, &graph);
  (void)hipStreamDestroy(st);
  if (err != CSA2_OK || ec != hipSuccess || !graph) {
    if (graph) (void)hipGraphDestroy(graph);
    return err != CSA2_OK ? err : CSA2_EHIP;
  }
  hipGraphExec_t exec = nullptr;
  if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return CSA2_EHIP;
  }
  csa2_schedule_t* sch = new (std::nothrow) csa2_schedule_t{graph, exec};
  if (!sch) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return CSA2_EHIP;
  }
  *out = sch;
  return CSA2_OK;
}

int csa2_schedule_launch(csa2_schedule_t* sch, void* stream) {
  if (!sch) return CSA2_EINVAL;
  return hipGraphLaunch(sch->exec, (hipStream_t)stream) == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

void csa2_schedule_destroy(csa2_schedule_t* sch) {
  if (!sch) return;
  (void)hipGraphExecDestroy(sch->exec);
  (void)hipGraphDestroy(sch->graph);
  delete sch;
}

}  // extern "C"
