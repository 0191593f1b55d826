// Host-side launchers behind the C ABI (csa2.h).  Each returns a CSA2_* code.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

// Tokens per entry of a cache (0 in the descriptor means 2), and the shift that
// turns a token count into the visible entry count: n_vis = tokens >> shift.
inline int cache_ratio(const csa2_cache_t& c) { return c.ratio == 1 ? 1 : 2; }
inline int vis_shift(const csa2_cache_t& c) { return c.ratio == 1 ? 0 : 1; }

// Workspace layout of csa2_index_full, shared by the size query and the launcher.
struct IndexFullPlan {
  int chunk;          // entries scored by one workgroup (power of two, >= topk)
  int n_chunks;       // chunks covering max_nvis entries
  int max_blocks;     // candidate blocks covering max_nvis entries
  int group;          // chunks merged per group before the final merge (0: no groups)
  int n_groups;
  size_t off_cand_key, off_cand_idx, off_cand_cnt, off_blockmax;
  size_t off_grp_key, off_grp_idx, off_grp_cnt, total;
};
// max_nvis: the most entries any sequence has visible (max_ctx >> vis_shift).
IndexFullPlan plan_index_full(int B, int64_t max_nvis, int topk, int pool_blocks, int cand_block);

int launch_write_kv(const csa2_cache_t& c, int B, const int32_t* start_tok, int T_new,
                    const uint16_t* x, const uint16_t* w, const uint16_t* k_idx, hipStream_t s);
// The write with the indexer key projected from each entry by the bf16 weights
// w_proj [64][512] instead of taken from the caller.
int launch_write_kv_proj(const csa2_cache_t& c, int B, const int32_t* start_tok, int T_new,
                         const uint16_t* x, const uint16_t* w, const uint16_t* w_proj, hipStream_t s);
// HISA block summaries of c's indexer keys into blocks' key arrays (blocks of
// cand_block entries): per sequence, blocks blk_first[b] .. +n_span-1, or all of them
// (n_span from max_ctx) when blk_first is null.
int launch_block_keys(const csa2_cache_t& c, const csa2_cache_t& blocks, int B, const int32_t* ctx_len,
                      int64_t max_ctx, int cand_block, const int32_t* blk_first, int n_span, int32_t* n_blocks_out,
                      hipStream_t s);
int launch_debug_gather(const csa2_cache_t& c, int B, const int32_t* idx, int n, float* out_lat,
                        float* out_idx, hipStream_t s);
int launch_index_full(const csa2_cache_t& c, int B, const int32_t* ctx_len, int64_t max_ctx,
                      const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                      int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, hipStream_t s);
// The step's write (as launch_write_kv) and the Full selection (as launch_index_full)
// in one launch: the scan stores each written entry that it streams before reading
// it, so the selection is the one the two calls give in that order.
int launch_write_index_full(const csa2_cache_t& c, int B, const int32_t* start_tok, int T_new, const uint16_t* x,
                            const uint16_t* w, const uint16_t* k_idx, const int32_t* ctx_len, int64_t max_ctx,
                            const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                            int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, hipStream_t s);
// Reindex: with a workspace of reindex_ws(B) bytes the pool is scored by many
// workgroups per sequence and selected by a second kernel; without one, by one
// workgroup per sequence.
size_t reindex_ws(int B);
int launch_reindex(const csa2_cache_t& c, int B, const int32_t* ctx_len, const uint16_t* q_idx,
                   const uint16_t* w_idx, const int32_t* pool, int pool_blocks, int cand_block,
                   int topk, int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t s);
// Sparse decode needs no workspace (sparse_decode_ws returns 0; the ABI keeps the
// argument): launches with few (query, head group) pairs split the output dims, not
// the rows, over several workgroups.
size_t sparse_decode_ws(int B, int H, int topk);
int launch_sparse_decode(const csa2_cache_t& c, int B, int H, const int32_t* ctx_len,
                         const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* swa,
                         int W, float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                         hipStream_t s);
// The attention kernel for B*C queries: C = 1 and prefill = false is the decode
// call; prefill = true reads query positions as len[b] + chunk index and window
// rows from a [B][W-1+C][512] array.  ws is unused.
int launch_gather_attention(const csa2_cache_t& c, int B, int C, int H, const int32_t* len, bool prefill,
                            const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* win,
                            int W, float sm_scale, uint16_t* out, float* lse, hipStream_t s,
                            void* ws = nullptr, size_t ws_bytes = 0);
// The batched attention kernels (attention_batch.hip), for launches with many
// (query, head group) pairs; same arguments and result as launch_gather_attention.
int launch_attention_batch(const csa2_cache_t& c, int B, int C, int H, const int32_t* len, bool prefill,
                           const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* win, int W,
                           float sm_scale, uint16_t* out, float* lse, hipStream_t s);
bool attention_batch_ready();
size_t prefill_ws(int B, int H, int64_t max_ctx, int topk, int C);
int launch_prefill_chunk(const csa2_cache_t& c, int B, int H, const int32_t* prior_len,
                         int64_t max_ctx, int C, const uint16_t* q, const uint16_t* q_idx,
                         const uint16_t* w_idx, const uint16_t* local, int W, int topk,
                         float sm_scale, uint16_t* out, int32_t* topk_idx, void* ws, hipStream_t s);

// Kernel attributes (dynamic LDS limits) set once per process; the schedule runner
// calls these before a stream capture so that no attribute call happens inside it.
bool index_kernels_ready();
bool attention_kernels_ready();

inline int hip_status() {
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

}  // namespace csa2
