// Indexer: Full-mode scan with top-K and HSI block maxima, the cross-chunk merge
// and pool selection, and Reindex over the candidate pool.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §2.3.1 (indexer
// query x indexer key scores every main entry, top-K per query), §2.3.2 (Full /
// Reindex modes), §2.3.4 (HSI: block maxima of the Full scores, newest block forced
// in, top blocks form the pool; Reindex scores only the pool; the Full scan over all
// visible entries is the remaining linear cost).  Score s_j = sum_h w_h *
// ReLU(q_h . k_j) over 4 heads (the pages give no formula; this is the library's).
//
// Full scan (index_scan_kernel): one workgroup per (sequence, chunk of CH entries).
// Each wave streams 16-entry groups of FP4 keys straight from the paged cache
// (8 bytes per lane, a wave covers 512 contiguous bytes), converts them to bf16
// with the hardware FP4 convert (scale folded in, exact) and scores the group with
// two 16x16x32 bf16 MFMAs: A = the 4 indexer heads (rows 4..15 zero), B = 16 keys.
// Lanes 0..15 then hold the 4 head dots of one entry each and form the score
// without any cross-lane reduction.  Scores never leave LDS: after the chunk is
// scored, the workgroup writes the block maxima (for the pool) and an exact local
// top-K (select.h) as (key, entry) candidates in entry order.  The global top-K is
// a subset of the union of the local top-Ks, so the merge is exact.
#include "common.h"
#include "internal.h"
#include "select.h"

namespace csa2 {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanR = 8;            // histogram replicas in the scan kernel
constexpr int kMergeThreads = 1024;
constexpr int kMergeR = 16;
constexpr int kMergeCap = 32768;     // keys the merge / pool workgroup holds in LDS
constexpr int kReindexThreads = 512;
constexpr int kReindexR = 16;
constexpr int kReindexCap = 16384;

__device__ __forceinline__ int n_visible_entries(const int32_t* ctx_len, int b, int64_t max_ctx) {
  int64_t L = ctx_len[b];
  if (L < 0) L = 0;
  if (L > max_ctx) L = max_ctx;
  return (int)(L >> 1);
}

// A-operand of the indexer MFMA: lane (m = l%16, g = l/16) holds head m's dims
// 8*(2g+s) .. +7 for k-step s; heads 4..15 are zero.
__device__ __forceinline__ void load_q_frags(const uint16_t* __restrict__ q_idx, int b, bf16x8& a0,
                                             bf16x8& a1) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
  if (m < CSA2_H_INDEX) {
    const uint16_t* q = q_idx + ((int64_t)b * CSA2_H_INDEX + m) * CSA2_D_INDEX + 16 * g;
    v0 = *reinterpret_cast<const u32x4*>(q);
    v1 = *reinterpret_cast<const u32x4*>(q + 8);
  }
  a0 = __builtin_bit_cast(bf16x8, v0);
  a1 = __builtin_bit_cast(bf16x8, v1);
}

// Score 16 entries whose codes (8 bytes at dims 16g..16g+15 of entry l%16) and
// scale are already in registers.  Returns the score in lanes 0..15.
__device__ __forceinline__ float score16(u32x2 codes, uint32_t scale_byte, bf16x8 a0, bf16x8 a1,
                                         const float (&wh)[4]) {
  const float sc = e8m0_scale(scale_byte);
  u32x4 lo, hi;
  lo.x = fp4x2_to_bf16x2<0>(codes.x, sc);
  lo.y = fp4x2_to_bf16x2<1>(codes.x, sc);
  lo.z = fp4x2_to_bf16x2<2>(codes.x, sc);
  lo.w = fp4x2_to_bf16x2<3>(codes.x, sc);
  hi.x = fp4x2_to_bf16x2<0>(codes.y, sc);
  hi.y = fp4x2_to_bf16x2<1>(codes.y, sc);
  hi.z = fp4x2_to_bf16x2<2>(codes.y, sc);
  hi.w = fp4x2_to_bf16x2<3>(codes.y, sc);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, __builtin_bit_cast(bf16x8, lo), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, __builtin_bit_cast(bf16x8, hi), acc, 0, 0, 0);
  // lanes 0..15: acc[i] = head i . key(l%16)
  return wh[0] * fmaxf(acc[0], 0.f) + wh[1] * fmaxf(acc[1], 0.f) + wh[2] * fmaxf(acc[2], 0.f) +
         wh[3] * fmaxf(acc[3], 0.f);
}

struct ScanArgs {
  const uint8_t* idx_codes;
  const uint8_t* idx_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* ctx_len;
  int64_t max_ctx;
  const uint16_t* q_idx;
  const uint16_t* w_idx;
  int topk, chunk, n_chunks, cand_block, want_blocks, max_blocks;
  uint32_t* cand_key;
  int32_t* cand_idx;
  int32_t* cand_cnt;
  uint32_t* block_max;
};

__global__ __launch_bounds__(kScanThreads) void index_scan_kernel(ScanArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                          // [chunk]
  uint32_t* hist = smem + a.chunk;                // [256 * R]
  uint32_t* misc = hist + 256 * kScanR;           // [512]
  const int b = blockIdx.x / a.n_chunks;
  const int c = blockIdx.x - b * a.n_chunks;
  const int n_vis = n_visible_entries(a.ctx_len, b, a.max_ctx);
  const int e0 = c * a.chunk;
  const int64_t slot = (int64_t)b * a.n_chunks + c;
  if (e0 >= n_vis) {
    if (threadIdx.x == 0) a.cand_cnt[slot] = 0;
    return;
  }
  const int n_in = min(a.chunk, n_vis - e0);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n_grp = (n_in + 15) >> 4;

  bf16x8 a0, a1;
  load_q_frags(a.q_idx, b, a0, a1);
  float wh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wh[h] = bf16_to_f32(a.w_idx[b * CSA2_H_INDEX + h]);

  const int n = lane & 15, g = lane >> 4;
  // Each wave scores groups wid, wid+4, ...; four groups per step keep 4 loads in flight.
  constexpr int U = 4;
  for (int gb = wid * U; gb < n_grp; gb += 4 * U) {
    u32x2 cd[U];
    uint32_t sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int grp = gb + u;
      const int e = e0 + grp * 16 + n;           // this lane's entry
      cd[u] = u32x2{0u, 0u};
      sb[u] = 0u;
      if (grp < n_grp && e < n_vis) {
        const int page = page_of(a.block_table, a.max_pages, a.n_pages, b, e);
        if (page >= 0) {
          const int64_t row = (int64_t)page * CSA2_PAGE + (e & (CSA2_PAGE - 1));
          cd[u] = *reinterpret_cast<const u32x2*>(a.idx_codes + row * CSA2_IDX_CODE_BYTES + 8 * g);
          sb[u] = a.idx_scales[row * CSA2_IDX_SCALE_BYTES + (g >> 1)];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int grp = gb + u;
      if (grp >= n_grp) break;                    // wave-uniform
      const float s = score16(cd[u], sb[u], a0, a1, wh);
      const int le = grp * 16 + n;
      if (lane < 16) keys[le] = (le < n_in) ? score_key(s) : 0u;
    }
  }
  __syncthreads();

  // HSI block maxima of this chunk (as keys): block k covers entries k*cb .. +cb-1.
  if (a.want_blocks) {
    const int cb = a.cand_block;
    const int nb = (n_in + cb - 1) / cb;
    const int blk0 = e0 / cb;
    for (int k = threadIdx.x; k < nb; k += kScanThreads) {
      uint32_t m = 0u;
      const int lo = k * cb, hi = min(n_in, lo + cb);
      for (int e = lo; e < hi; ++e) m = max(m, keys[e]);
      a.block_max[(int64_t)b * a.max_blocks + blk0 + k] = m;
    }
  }

  const SelectResult sr = block_select<kScanThreads, kScanR>(keys, n_in, a.topk, SelectSmem{hist, misc});
  uint32_t* ck = a.cand_key + slot * a.topk;
  int32_t* ci = a.cand_idx + slot * a.topk;
  block_emit_ordered<kScanThreads>(keys, n_in, sr, misc + 256 + 8, [&](int v, uint32_t pos) {
    ck[pos] = keys[v];
    ci[pos] = e0 + v;
  });
  if (threadIdx.x == 0) a.cand_cnt[slot] = (int32_t)sr.count;
}

struct MergeArgs {
  const int32_t* ctx_len;
  int64_t max_ctx;
  int topk, chunk, n_chunks, cand_block, pool_blocks, max_blocks;
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  const int32_t* cand_cnt;
  const uint32_t* block_max;
  int32_t* topk_idx;
  int32_t* pool;
};

// blockIdx.y == 0: top-K over the chunk candidates; == 1: HSI pool over block maxima.
__global__ __launch_bounds__(kMergeThreads) void index_merge_kernel(MergeArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                          // [kMergeCap]
  uint32_t* hist = smem + kMergeCap;              // [256 * R]
  uint32_t* misc = hist + 256 * kMergeR;          // [512]
  const int b = blockIdx.x;
  const int n_vis = n_visible_entries(a.ctx_len, b, a.max_ctx);
  const int tid = threadIdx.x;
  if (blockIdx.y == 0) {
    const int nc = (n_vis + a.chunk - 1) / a.chunk;
    const int N = nc * a.topk;                    // virtual slot v = chunk * topk + i
    for (int v = tid; v < N; v += kMergeThreads) {
      const int cch = v / a.topk, i = v - cch * a.topk;
      const int64_t slot = (int64_t)b * a.n_chunks + cch;
      keys[v] = (i < a.cand_cnt[slot]) ? a.cand_key[slot * a.topk + i] : 0u;
    }
    __syncthreads();
    const SelectResult sr = block_select<kMergeThreads, kMergeR>(keys, N, a.topk, SelectSmem{hist, misc});
    int32_t* out = a.topk_idx + (int64_t)b * a.topk;
    block_emit_ordered<kMergeThreads>(keys, N, sr, misc + 256 + 8, [&](int v, uint32_t pos) {
      const int cch = v / a.topk, i = v - cch * a.topk;
      out[pos] = a.cand_idx[((int64_t)b * a.n_chunks + cch) * a.topk + i];
    });
    for (int p = (int)sr.count + tid; p < a.topk; p += kMergeThreads) out[p] = -1;
  } else {
    const int cb = a.cand_block;
    const int nb = (n_vis + cb - 1) / cb;
    const uint32_t* bm = a.block_max + (int64_t)b * a.max_blocks;
    for (int v = tid; v < nb; v += kMergeThreads) keys[v] = bm[v];
    __syncthreads();
    if (tid == 0 && nb > 0) keys[nb - 1] = 0xffffffffu;   // newest visible block: +inf
    __syncthreads();
    const SelectResult sr = block_select<kMergeThreads, kMergeR>(keys, nb, a.pool_blocks, SelectSmem{hist, misc});
    int32_t* out = a.pool + (int64_t)b * a.pool_blocks;
    block_emit_ordered<kMergeThreads>(keys, nb, sr, misc + 256 + 8,
                                      [&](int v, uint32_t pos) { out[pos] = v; });
    for (int p = (int)sr.count + tid; p < a.pool_blocks; p += kMergeThreads) out[p] = -1;
  }
}

struct ReindexArgs {
  const uint8_t* idx_codes;
  const uint8_t* idx_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* ctx_len;
  const uint16_t* q_idx;
  const uint16_t* w_idx;
  const int32_t* pool;
  int pool_blocks, cand_block, topk;
  int32_t* topk_idx;
};

// One workgroup per sequence: score the pool's entries (slot v = p*cb + i is entry
// pool[p]*cb + i), keep the top-K.  The pool is ascending, so slot order is entry order.
__global__ __launch_bounds__(kReindexThreads) void reindex_kernel(ReindexArgs a) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem;                          // [pool_blocks * cb]
  uint32_t* hist = smem + kReindexCap;
  uint32_t* misc = hist + 256 * kReindexR;
  const int b = blockIdx.x;
  int64_t L = a.ctx_len[b];
  if (L < 0) L = 0;
  const int64_t n_vis = L >> 1;
  const int cb = a.cand_block;
  const int N = a.pool_blocks * cb;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int NW = kReindexThreads / 64;
  const int n = lane & 15, g = lane >> 4;
  bf16x8 a0, a1;
  load_q_frags(a.q_idx, b, a0, a1);
  float wh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wh[h] = bf16_to_f32(a.w_idx[b * CSA2_H_INDEX + h]);
  const int32_t* pool = a.pool + (int64_t)b * a.pool_blocks;
  const int n_grp = (N + 15) >> 4;
  constexpr int U = 4;
  for (int gb = wid * U; gb < n_grp; gb += NW * U) {
    u32x2 cd[U];
    uint32_t sb[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = (gb + u) * 16 + n;
      cd[u] = u32x2{0u, 0u};
      sb[u] = 0u;
      ok[u] = false;
      if (v < N) {
        const int blk = pool[v / cb];
        const int64_t e = (int64_t)blk * cb + (v % cb);
        if (blk >= 0 && e < n_vis) {
          const int page = page_of(a.block_table, a.max_pages, a.n_pages, b, (int)e);
          if (page >= 0) {
            const int64_t row = (int64_t)page * CSA2_PAGE + (e & (CSA2_PAGE - 1));
            cd[u] = *reinterpret_cast<const u32x2*>(a.idx_codes + row * CSA2_IDX_CODE_BYTES + 8 * g);
            sb[u] = a.idx_scales[row * CSA2_IDX_SCALE_BYTES + (g >> 1)];
            ok[u] = true;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int grp = gb + u;
      if (grp >= n_grp) break;
      const float s = score16(cd[u], sb[u], a0, a1, wh);
      // entry validity lives in the lane that loaded it (lane n + 16*g); lanes 0..15 hold g = 0
      const int v = grp * 16 + n;
      if (lane < 16 && v < N) keys[v] = ok[u] ? score_key(s) : 0u;
    }
  }
  __syncthreads();
  const SelectResult sr = block_select<kReindexThreads, kReindexR>(keys, N, a.topk, SelectSmem{hist, misc});
  int32_t* out = a.topk_idx + (int64_t)b * a.topk;
  block_emit_ordered<kReindexThreads>(keys, N, sr, misc + 256 + 8, [&](int v, uint32_t pos) {
    out[pos] = pool[v / cb] * cb + (v % cb);
  });
  for (int p = (int)sr.count + threadIdx.x; p < a.topk; p += kReindexThreads) out[p] = -1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Kernels here take up to ~150 KB of dynamic LDS (gfx950 has 160 KB per CU); raise
// each kernel's limit once per process.
bool lds_limits_set() {
  static const bool ok = [] {
    bool r = hipFuncSetAttribute(reinterpret_cast<const void*>(index_scan_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    r = r && hipFuncSetAttribute(reinterpret_cast<const void*>(index_merge_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    r = r && hipFuncSetAttribute(reinterpret_cast<const void*>(reindex_kernel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    return r;
  }();
  return ok;
}

}  // namespace

IndexFullPlan plan_index_full(int B, int64_t max_ctx, int topk, int pool_blocks, int cand_block) {
  (void)cand_block;
  IndexFullPlan p{};
  const int64_t max_nvis = max_ctx / 2;
  int ch = 4096;
  while (ch < topk) ch *= 2;
  int64_t nc = (max_nvis + ch - 1) / ch;
  while (nc * topk > kMergeCap && ch < 16384) {
    ch *= 2;
    nc = (max_nvis + ch - 1) / ch;
  }
  if (nc < 1) nc = 1;
  if (nc * topk > kMergeCap || ch > 16384) return p;      // chunk = 0: unsupported
  // pool: block maxima sized for the smallest block (1 entry) so any cand_block fits
  const int64_t max_blocks = pool_blocks > 0 ? std::max<int64_t>(max_nvis, 1) : 0;
  if (pool_blocks > 0 && (max_nvis + 7) / 8 > kMergeCap) return p;
  p.chunk = ch;
  p.n_chunks = (int)nc;
  p.max_blocks = (int)max_blocks;
  size_t off = 0;
  p.off_cand_key = off;
  off = align256(off + (size_t)B * nc * topk * 4);
  p.off_cand_idx = off;
  off = align256(off + (size_t)B * nc * topk * 4);
  p.off_cand_cnt = off;
  off = align256(off + (size_t)B * nc * 4);
  p.off_blockmax = off;
  off = align256(off + (size_t)B * max_blocks * 4);
  p.total = off;
  return p;
}

int launch_index_full(const csa2_cache_t& c, int B, const int32_t* ctx_len, int64_t max_ctx,
                      const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                      int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, hipStream_t s) {
  const IndexFullPlan p = plan_index_full(B, max_ctx, topk, pool_blocks, cand_block);
  if (p.chunk == 0) return CSA2_EUNSUPPORTED;
  if (pool_blocks > 0 && (max_ctx / 2 + cand_block - 1) / cand_block > kMergeCap) return CSA2_EUNSUPPORTED;
  if (!lds_limits_set()) return CSA2_EHIP;
  uint8_t* w = static_cast<uint8_t*>(ws);
  ScanArgs sa;
  sa.idx_codes = c.idx_codes;
  sa.idx_scales = c.idx_scales;
  sa.block_table = c.block_table;
  sa.n_pages = c.n_pages;
  sa.max_pages = c.max_pages;
  sa.ctx_len = ctx_len;
  sa.max_ctx = max_ctx;
  sa.q_idx = q_idx;
  sa.w_idx = w_idx;
  sa.topk = topk;
  sa.chunk = p.chunk;
  sa.n_chunks = p.n_chunks;
  sa.cand_block = cand_block;
  sa.want_blocks = pool_blocks > 0;
  sa.max_blocks = p.max_blocks;
  sa.cand_key = reinterpret_cast<uint32_t*>(w + p.off_cand_key);
  sa.cand_idx = reinterpret_cast<int32_t*>(w + p.off_cand_idx);
  sa.cand_cnt = reinterpret_cast<int32_t*>(w + p.off_cand_cnt);
  sa.block_max = reinterpret_cast<uint32_t*>(w + p.off_blockmax);
  const size_t scan_lds = (size_t)(p.chunk + 256 * kScanR + 512) * 4;
  const int64_t grid = (int64_t)B * p.n_chunks;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  hipLaunchKernelGGL(index_scan_kernel, dim3((unsigned)grid), dim3(kScanThreads), scan_lds, s, sa);
  if (hip_status() != CSA2_OK) return CSA2_EHIP;

  MergeArgs ma;
  ma.ctx_len = ctx_len;
  ma.max_ctx = max_ctx;
  ma.topk = topk;
  ma.chunk = p.chunk;
  ma.n_chunks = p.n_chunks;
  ma.cand_block = cand_block;
  ma.pool_blocks = pool_blocks;
  ma.max_blocks = p.max_blocks;
  ma.cand_key = sa.cand_key;
  ma.cand_idx = sa.cand_idx;
  ma.cand_cnt = sa.cand_cnt;
  ma.block_max = sa.block_max;
  ma.topk_idx = topk_idx;
  ma.pool = pool;
  const size_t merge_lds = (size_t)(kMergeCap + 256 * kMergeR + 512) * 4;
  hipLaunchKernelGGL(index_merge_kernel, dim3(B, pool_blocks > 0 ? 2 : 1), dim3(kMergeThreads),
                     merge_lds, s, ma);
  return hip_status();
}

int launch_reindex(const csa2_cache_t& c, int B, const int32_t* ctx_len, const uint16_t* q_idx,
                   const uint16_t* w_idx, const int32_t* pool, int pool_blocks, int cand_block,
                   int topk, int32_t* topk_idx, hipStream_t s) {
  if ((int64_t)pool_blocks * cand_block > kReindexCap) return CSA2_EUNSUPPORTED;
  if (!lds_limits_set()) return CSA2_EHIP;
  ReindexArgs ra;
  ra.idx_codes = c.idx_codes;
  ra.idx_scales = c.idx_scales;
  ra.block_table = c.block_table;
  ra.n_pages = c.n_pages;
  ra.max_pages = c.max_pages;
  ra.ctx_len = ctx_len;
  ra.q_idx = q_idx;
  ra.w_idx = w_idx;
  ra.pool = pool;
  ra.pool_blocks = pool_blocks;
  ra.cand_block = cand_block;
  ra.topk = topk;
  ra.topk_idx = topk_idx;
  const size_t lds = (size_t)(kReindexCap + 256 * kReindexR + 512) * 4;
  hipLaunchKernelGGL(reindex_kernel, dim3(B), dim3(kReindexThreads), lds, s, ra);
  return hip_status();
}

}  // namespace csa2
