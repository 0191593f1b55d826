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
// Each wave streams whole 64-entry pages of FP4 keys straight from the paged cache
// with buffer loads off a per-page descriptor (8 bytes per lane and group of 16
// entries, a wave covers 512 contiguous bytes), converts them to bf16 with the
// hardware FP4 convert (scale folded in, exact) and scores a page with eight
// 16x16x32 bf16 MFMAs into one accumulator: group u of the page meets the 4
// indexer heads placed in rows 4u..4u+3 (the other rows zero), so lane l ends with
// the 4 head dots of entry l and forms its score without any cross-lane reduction,
// and the ReLU, weighting and key conversion run once per page, not once per group.
// Measured on the MI355X at 8 x 524,288 entries, this cut the vector ALU work of
// the stream by two thirds, which had bound it as much as the HBM reads.
// Scores never leave LDS: after the chunk is
// scored, the workgroup writes the block maxima (for the pool) and an exact local
// top-K (select.h) as (key, entry) candidates in entry order.  The global top-K is
// a subset of the union of the local top-Ks, so the merge is exact.
#include "common.h"
#include "entry_write.h"
#include "internal.h"
#include "select.h"

namespace csa2 {
namespace {

constexpr int kScanThreads = 512;
constexpr int kScanAhead = 2;        // pages a scan wave keeps in flight beyond the one it scores
constexpr int kScanMaxWrites = 2;    // entries per sequence up to which the scan does the step's write
constexpr int kReindexRound = 8;     // groups of 16 pool slots a reindex wave loads before scoring them
constexpr int kMergeThreads = 1024;
constexpr int kMergeCap = 32768;     // keys the merge / pool workgroup selects from
constexpr int kReindexThreads = 512;
constexpr int kReindexCap = 16384;

// Entries visible to a decode query of ctx_len[b] tokens: one per `ratio` tokens,
// given as the shift vshift (1 for ratio 2, 0 for ratio 1).
__device__ __forceinline__ int n_visible_entries(const int32_t* ctx_len, int b, int64_t max_ctx, int vshift) {
  int64_t L = ctx_len[b];
  if (L < 0) L = 0;
  if (L > max_ctx) L = max_ctx;
  return (int)(L >> vshift);
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
  return wh[0] * relu0(acc[0]) + wh[1] * relu0(acc[1]) + wh[2] * relu0(acc[2]) + wh[3] * relu0(acc[3]);
}

// A-operands that score a whole 64-entry page with one accumulator: group u (entries
// 16u..16u+15) is multiplied with the 4 heads placed in rows 4u..4u+3 and zero rows
// elsewhere, so the eight MFMAs of a page add into one register set and each group
// fills only its own 16 lanes.  Lane (m = l%16, g = l/16) of a[u][s] holds head m%4's
// dims 8*(2g+s) .. +7 when m/4 == u, zero otherwise.
__device__ __forceinline__ void load_q_frags_page(const uint16_t* __restrict__ q_idx, int b,
                                                  bf16x8 (&a)[4][2]) {
  static_assert(CSA2_H_INDEX == 4, "four groups of four heads fill the 16 rows");
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const uint16_t* q = q_idx + ((int64_t)b * CSA2_H_INDEX + (m & 3)) * CSA2_D_INDEX + 16 * g;
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(q);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(q + 8);
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    a[u][0] = __builtin_bit_cast(bf16x8, (m >> 2) == u ? v0 : z);
    a[u][1] = __builtin_bit_cast(bf16x8, (m >> 2) == u ? v1 : z);
  }
}

// Scores of the 64 entries of a page: cd[u] holds the 8 code bytes at dims
// 16g..16g+15 of entry 16u + l%16 and sb[u] that entry's scale byte for those dims.
// Lane l returns the score of entry l.  A lane's own group adds its two products to
// an accumulator that holds +0, and the other groups add exact zeros, so the score
// is the one a separate 16-entry product gives, bit for bit.
__device__ __forceinline__ float score_page(const u32x2 (&cd)[4], const uint32_t (&sb)[4],
                                            const bf16x8 (&a)[4][2], const float (&wh)[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float sc = e8m0_scale(sb[u]);
    u32x4 lo, hi;
    lo.x = fp4x2_to_bf16x2<0>(cd[u].x, sc);
    lo.y = fp4x2_to_bf16x2<1>(cd[u].x, sc);
    lo.z = fp4x2_to_bf16x2<2>(cd[u].x, sc);
    lo.w = fp4x2_to_bf16x2<3>(cd[u].x, sc);
    hi.x = fp4x2_to_bf16x2<0>(cd[u].y, sc);
    hi.y = fp4x2_to_bf16x2<1>(cd[u].y, sc);
    hi.z = fp4x2_to_bf16x2<2>(cd[u].y, sc);
    hi.w = fp4x2_to_bf16x2<3>(cd[u].y, sc);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][0], __builtin_bit_cast(bf16x8, lo), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][1], __builtin_bit_cast(bf16x8, hi), acc, 0, 0, 0);
  }
  return wh[0] * relu0(acc[0]) + wh[1] * relu0(acc[1]) + wh[2] * relu0(acc[2]) + wh[3] * relu0(acc[3]);
}

// Buffer descriptor of one page's bytes (raw buffer, dword 3 as gfx9 wants it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}

// Maxima of blocks of CB consecutive keys, from the keys in registers (thread t holds
// positions t*KPT .. +KPT-1): a thread holds KPT/CB whole blocks, or a block spans
// CB/KPT adjacent lanes.  Block k goes to bm[k] for k < nb.
template <int KPT, int CB>
__device__ __forceinline__ void block_maxima(const uint32_t (&kr)[KPT], uint32_t* __restrict__ bm, int nb) {
  if constexpr (CB <= KPT) {
#pragma unroll
    for (int j = 0; j < KPT; j += CB) {
      uint32_t m = kr[j];
#pragma unroll
      for (int i = 1; i < CB; ++i) m = max(m, kr[j + i]);
      const int k = (int)(threadIdx.x * (KPT / CB)) + j / CB;
      if (k < nb) bm[k] = m;
    }
  } else {
    constexpr int R = CB / KPT;   // lanes per block
    static_assert(R <= 64, "a block lies within a wave");
    uint32_t m = kr[0];
#pragma unroll
    for (int i = 1; i < KPT; ++i) m = max(m, kr[i]);
#pragma unroll
    for (int o = 1; o < R; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, kWave));
    const int k = (int)threadIdx.x / R;
    if ((threadIdx.x & (R - 1)) == 0 && k < nb) bm[k] = m;
  }
}

struct ScanArgs {
  const uint8_t* idx_codes;
  const uint8_t* idx_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* ctx_len;
  int64_t max_ctx;
  int vshift;            // token count -> visible entries: >> vshift
  const uint16_t* q_idx;
  const uint16_t* w_idx;
  int topk, n_chunks, cand_block, want_blocks, max_blocks;
  uint32_t* cand_key;
  int32_t* cand_idx;
  int32_t* cand_cnt;
  uint32_t* block_max;
  WriteArgs wr;          // the step's write, done by this launch (wr.x == nullptr: none)
};

// NT threads stream one chunk: 512, or 1024 when the grid leaves one workgroup per
// CU (twice the waves, so twice the key loads in flight per CU, for the same chunk).
template <int CHUNK, int NT = kScanThreads>
__global__ __launch_bounds__(NT) void index_scan_kernel(ScanArgs a) {
  constexpr int KPT = CHUNK / NT;
  extern __shared__ __align__(16) uint32_t smem[];
  uint32_t* keys = smem;                          // [CHUNK]
  uint32_t* hist = smem + CHUNK;                  // [kSelectHist]
  uint32_t* scratch = hist + kSelectHist;         // [kSelectScratch]
  const int b = blockIdx.x / a.n_chunks;
  const int c = blockIdx.x - b * a.n_chunks;
  const int n_vis = n_visible_entries(a.ctx_len, b, a.max_ctx, a.vshift);
  const int e0 = c * CHUNK;
  const int64_t slot = (int64_t)b * a.n_chunks + c;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  constexpr int NW = NT / 64;
  constexpr int NPW = CHUNK / CSA2_PAGE / NW;   // pages per wave

  // The step's write, when this launch performs it (the scan then sees the written
  // keys, as if the write had run first).  A visible written entry is stored by the
  // workgroup that streams it before its rows are read (below); the entries no chunk
  // streams are spread over all waves of the sequence's workgroups here.
  int wj0 = -1;
  if (a.wr.x != nullptr) {
    wj0 = write_first_entry(a.wr, b);
    if (wj0 >= 0) {
      const int stride = a.n_chunks * NW;
      for (int i = max(0, n_vis - wj0) + c * NW + wid; i < a.wr.half; i += stride)
        write_entry_wave(a.wr, b, i, lane);
    }
  }
  if (e0 >= n_vis) {
    if (threadIdx.x == 0) a.cand_cnt[slot] = 0;
    return;
  }
  const int n_in = min(CHUNK, n_vis - e0);
  const int n = lane & 15, g = lane >> 4;
  if (wj0 >= 0) {
    // the wave that streams a written entry's page stores the entry, and only that
    // wave waits for its stores before it issues its loads of those rows
    const int lo = max(wj0, e0 + wid * NPW * CSA2_PAGE);
    const int hi = min(min(wj0 + a.wr.half, e0 + (wid + 1) * NPW * CSA2_PAGE), n_vis);
    for (int j = lo; j < hi; ++j) write_entry_wave(a.wr, b, j - wj0, lane);
    if (lo < hi) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }

  bf16x8 aq[4][2];
  load_q_frags_page(a.q_idx, b, aq);
  float wh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wh[h] = bf16_to_f32(a.w_idx[b * CSA2_H_INDEX + h]);

  // Wave w streams the NPW pages [w*NPW, (w+1)*NPW) of the chunk, one page a round.
  // The page ids come first, with one vector load (lane k: the wave's page k).  A
  // round's loads are buffer loads from a descriptor of its page: the page base sits
  // in scalar registers and every lane's offsets are constants, so issuing a round
  // takes no vector ALU work.  LA rounds are in flight while one is scored.
  static_assert(NPW <= kWave && NPW * NW * CSA2_PAGE == CHUNK, "one page id per lane");
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  int pgv;
  {
    const int ew0 = e0 + wid * NPW * CSA2_PAGE;   // wave-uniform
    const int pi = (ew0 >> 6) + lane;
    const int p = bt[min(pi, a.max_pages - 1)];
    pgv = (lane < NPW && ew0 + CSA2_PAGE * lane < n_vis && pi < a.max_pages && p >= 0 && p < a.n_pages) ? p : -1;
  }
  // lane (n, g): code bytes 8g.. of entry 16u + n, scale byte g/2 of that entry
  const int voff_code = n * CSA2_IDX_CODE_BYTES + 8 * g;
  const int voff_scale = n * CSA2_IDX_SCALE_BYTES + (g >> 1);
  struct Round {
    u32x2 cd[4];
    uint32_t sb[4];
  };
  auto load_round = [&](int r, Round& R) {
    const int pg = __builtin_amdgcn_readlane(pgv, r);
    const int64_t pc = pg >= 0 ? pg : 0;   // absent page: page 0 is read, its keys dropped
    const __amdgpu_buffer_rsrc_t rc = page_rsrc(a.idx_codes + pc * (CSA2_PAGE * CSA2_IDX_CODE_BYTES),
                                                CSA2_PAGE * CSA2_IDX_CODE_BYTES);
    const __amdgpu_buffer_rsrc_t rs = page_rsrc(a.idx_scales + pc * (CSA2_PAGE * CSA2_IDX_SCALE_BYTES),
                                                CSA2_PAGE * CSA2_IDX_SCALE_BYTES);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      R.cd[u] = __builtin_amdgcn_raw_buffer_load_b64(rc, voff_code + u * 16 * CSA2_IDX_CODE_BYTES, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      R.sb[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff_scale + u * 16 * CSA2_IDX_SCALE_BYTES, 0, 0);
  };
  auto score_round = [&](int r, const Round& R) {
    const int le = (wid * NPW + r) * CSA2_PAGE;   // chunk position of the page's entry 0
    const bool present = __builtin_amdgcn_readlane(pgv, r) >= 0;
    const float s = score_page(R.cd, R.sb, aq, wh);
    keys[le + lane] = (present && le + lane < n_in) ? score_key(s) : 0u;   // absent page: no entry
  };
  constexpr int LA = kScanAhead;                 // rounds in flight beyond the one scored
  // A wave with no visible entry skips the stream (its keys are cleared below with the
  // chunk's tail).  Any other wave streams all its pages with no branch between a
  // round's loads and its scoring (entries past the end score to key 0).
  if (e0 + wid * NPW * CSA2_PAGE < n_vis) {
    Round rr[LA + 1];
#pragma unroll
    for (int i = 0; i < LA && i < NPW; ++i) load_round(i, rr[i]);
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
      if (i + LA < NPW) load_round(i + LA, rr[(i + LA) % (LA + 1)]);
      score_round(i, rr[i % (LA + 1)]);
    }
  }
  // tail of a partial chunk: keys of absent entries are 0
  for (int i = ((n_in + 15) & ~15) + threadIdx.x; i < CHUNK; i += NT) keys[i] = 0u;
  __syncthreads();

  uint32_t kr[KPT];
#pragma unroll
  for (int i = 0; i < KPT; i += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(keys + threadIdx.x * KPT + i);
    kr[i] = v.x;
    kr[i + 1] = v.y;
    kr[i + 2] = v.z;
    kr[i + 3] = v.w;
  }
  // HSI block maxima of this chunk (as keys): block k covers entries k*cb .. +cb-1;
  // keys past the chunk's entries are 0 and leave the maxima unchanged.
  if (a.want_blocks) {
    uint32_t* bm = a.block_max + (int64_t)b * a.max_blocks + e0 / a.cand_block;
    const int nb = (n_in + a.cand_block - 1) / a.cand_block;
    switch (a.cand_block) {
      case 1: block_maxima<KPT, 1>(kr, bm, nb); break;
      case 2: block_maxima<KPT, 2>(kr, bm, nb); break;
      case 4: block_maxima<KPT, 4>(kr, bm, nb); break;
      case 8: block_maxima<KPT, 8>(kr, bm, nb); break;
      case 16: block_maxima<KPT, 16>(kr, bm, nb); break;
      default: block_maxima<KPT, 32>(kr, bm, nb); break;
    }
  }
  const SelectResult sr = block_select<NT, KPT>(kr, a.topk, hist, scratch);
  uint32_t* ck = a.cand_key + slot * a.topk;
  int32_t* ci = a.cand_idx + slot * a.topk;
  const int p0 = threadIdx.x * KPT;
  block_emit<NT, KPT>(kr, sr, scratch, [&](int i, uint32_t pos) {
    ck[pos] = kr[i];
    ci[pos] = e0 + p0 + i;
  });
  // unused slots hold key 0 ("no entry"), so readers need not wait for the count
  for (int p = (int)sr.count + threadIdx.x; p < a.topk; p += NT) ck[p] = 0u;
  if (threadIdx.x == 0) a.cand_cnt[slot] = (int32_t)sr.count;
}

struct MergeArgs {
  const int32_t* ctx_len;
  int64_t max_ctx;
  int vshift;            // token count -> visible entries: >> vshift
  int topk, chunk, n_chunks, cand_block, pool_blocks, max_blocks;
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  const int32_t* cand_cnt;
  const uint32_t* block_max;
  int32_t* topk_idx;
  int32_t* pool;
};

// blockIdx.y == 0: top-K over the chunk candidates; == 1: HSI pool over block maxima.
// KPT (keys per thread) is the smallest of 4/8/16/32 that covers both key sets.
// A thread's run of KPT consecutive words v[i] = base[p0 + i] (p0 a multiple of KPT);
// words at or past n read as `fill`.  The run is read with 16-byte loads when it lies
// inside [0, n) and base is 16-byte aligned, else word by word: word loads with
// 4 * KPT bytes between lanes touched a cache line per lane and pair of loads.
template <int KPT, class T>
__device__ __forceinline__ void load_run(const T* base, int p0, int n, T fill, T (&v)[KPT]) {
  static_assert(KPT % 4 == 0 && sizeof(T) == 4, "runs of 4-byte words in 16-byte pieces");
  if ((reinterpret_cast<uintptr_t>(base) & 15) == 0 && p0 + KPT <= n) {
#pragma unroll
    for (int i = 0; i < KPT; i += 4) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(base + p0 + i);
      // value conversions: __builtin_bit_cast of a vector element miscompiles here
      // (every element read as .x)
      v[i] = (T)x.x;
      v[i + 1] = (T)x.y;
      v[i + 2] = (T)x.z;
      v[i + 3] = (T)x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) v[i] = p0 + i < n ? base[p0 + i] : fill;
  }
}

template <int KPT>
__global__ __launch_bounds__(kMergeThreads) void index_merge_kernel(MergeArgs a) {
  __shared__ __align__(16) uint32_t hist[kSelectHist];
  __shared__ uint32_t scratch[kSelectScratch];
  const int b = blockIdx.x;
  const int n_vis = n_visible_entries(a.ctx_len, b, a.max_ctx, a.vshift);
  const int tid = threadIdx.x;
  const int p0 = tid * KPT;
  uint32_t kr[KPT];
  if (blockIdx.y == 0) {
    // virtual position v = chunk * topk + i, in entry order
    const int nc = (n_vis + a.chunk - 1) / a.chunk;
    const int N = nc * a.topk;
    // unused candidate slots hold key 0; keys and ids are loaded together, one round trip
    const uint32_t* ckey = a.cand_key + (int64_t)b * a.n_chunks * a.topk;
    const int32_t* cidx = a.cand_idx + (int64_t)b * a.n_chunks * a.topk;
    int32_t id[KPT];
    load_run<KPT>(ckey, p0, N, 0u, kr);
    load_run<KPT>(cidx, p0, N, -1, id);
    const SelectResult sr = block_select<kMergeThreads, KPT>(kr, a.topk, hist, scratch);
    int32_t* out = a.topk_idx + (int64_t)b * a.topk;
    block_emit<kMergeThreads, KPT>(kr, sr, scratch, [&](int i, uint32_t pos) { out[pos] = id[i]; });
    for (int p = (int)sr.count + tid; p < a.topk; p += kMergeThreads) out[p] = -1;
  } else {
    // The newest visible block ranks first (its maximum counts as +inf) and has the
    // largest id, so it is the last entry of the ascending pool; the other
    // pool_blocks - 1 slots are the best of the older blocks.
    const int cb = a.cand_block;
    const int nb = (n_vis + cb - 1) / cb;
    const uint32_t* bm = a.block_max + (int64_t)b * a.max_blocks;
    load_run<KPT>(bm, p0, nb - 1, 0u, kr);
    int32_t* out = a.pool + (int64_t)b * a.pool_blocks;
    uint32_t n_old = 0;
    if (nb > 1 && a.pool_blocks > 1) {                                // uniform over the block
      const SelectResult sr = block_select<kMergeThreads, KPT>(kr, a.pool_blocks - 1, hist, scratch);
      block_emit<kMergeThreads, KPT>(kr, sr, scratch, [&](int i, uint32_t pos) { out[pos] = p0 + i; });
      n_old = sr.count;
    }
    const int n_out = nb > 0 ? (int)n_old + 1 : 0;
    if (tid == 0 && nb > 0) out[n_old] = nb - 1;
    for (int p = n_out + tid; p < a.pool_blocks; p += kMergeThreads) out[p] = -1;
  }
}

struct GroupArgs {
  const int32_t* ctx_len;
  int64_t max_ctx;
  int vshift;            // token count -> visible entries: >> vshift
  int topk, chunk, n_chunks, group, n_groups;
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  const int32_t* cand_cnt;
  uint32_t* grp_key;
  int32_t* grp_idx;
  int32_t* grp_cnt;
};

// Long contexts: the candidates of `group` consecutive chunks are reduced to their
// top-K first (one workgroup per sequence and group), in the chunk-candidate format,
// so the final merge selects from n_groups * K keys instead of n_chunks * K.  Exact:
// the global top-K is contained in the union of the groups' top-Ks, and the kept
// keys stay in entry order.
template <int KPT>
__global__ __launch_bounds__(kMergeThreads) void index_group_kernel(GroupArgs a) {
  __shared__ __align__(16) uint32_t hist[kSelectHist];
  __shared__ uint32_t scratch[kSelectScratch];
  const int b = blockIdx.x, grp = blockIdx.y;
  const int n_vis = n_visible_entries(a.ctx_len, b, a.max_ctx, a.vshift);
  const int nc = (n_vis + a.chunk - 1) / a.chunk;
  const int c0 = grp * a.group;
  const int64_t gslot = (int64_t)b * a.n_groups + grp;
  if (c0 >= nc) {
    if (threadIdx.x == 0) a.grp_cnt[gslot] = 0;
    return;
  }
  const int N = min(a.group, nc - c0) * a.topk;
  const int tid = threadIdx.x;
  const int p0 = tid * KPT;
  const int64_t cbase = (int64_t)b * a.n_chunks + c0;
  const uint32_t* ckey = a.cand_key + cbase * a.topk;
  // unused candidate slots hold key 0; keys and ids are loaded together, one round trip
  const int32_t* cidx = a.cand_idx + cbase * a.topk;
  uint32_t kr[KPT];
  int32_t id[KPT];
  load_run<KPT>(ckey, p0, N, 0u, kr);
  load_run<KPT>(cidx, p0, N, -1, id);
  const SelectResult sr = block_select<kMergeThreads, KPT>(kr, a.topk, hist, scratch);
  uint32_t* gk = a.grp_key + gslot * a.topk;
  int32_t* gi = a.grp_idx + gslot * a.topk;
  block_emit<kMergeThreads, KPT>(kr, sr, scratch, [&](int i, uint32_t pos) {
    gk[pos] = kr[i];
    gi[pos] = id[i];
  });
  for (int p = (int)sr.count + tid; p < a.topk; p += kMergeThreads) gk[p] = 0u;   // key 0: no entry
  if (tid == 0) a.grp_cnt[gslot] = (int32_t)sr.count;
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
  int vshift;            // token count -> visible entries: >> vshift
  int cb_shift;          // log2(cand_block): slot v lies in pool block v >> cb_shift
};

// One workgroup per sequence: score the pool's entries (slot v = p*cb + i is entry
// pool[p]*cb + i), keep the top-K.  The pool is ascending, so slot order is entry order.
// KPT (keys per thread) is the smallest of 8/16/32 that covers the pool.
template <int KPT>
__global__ __launch_bounds__(kReindexThreads) void reindex_kernel(ReindexArgs a) {
  constexpr int kCap = KPT * kReindexThreads;
  extern __shared__ __align__(16) uint32_t smem[];
  uint32_t* keys = smem;                          // [kCap]
  uint32_t* hist = smem + kCap;
  uint32_t* scratch = hist + kSelectHist;
  const int b = blockIdx.x;
  int64_t L = a.ctx_len[b];
  if (L < 0) L = 0;
  const int64_t n_vis = L >> a.vshift;
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
  // Resolve every pool slot to its cache row (or -1) first, into the key array.
  int32_t* rowid = reinterpret_cast<int32_t*>(keys);
  for (int v = threadIdx.x; v < N; v += kReindexThreads) {
    const int blk = pool[v >> a.cb_shift];
    const int64_t e = (int64_t)blk * cb + (v & (cb - 1));
    int32_t rid = -1;
    if (blk >= 0 && e < n_vis) {
      const int page = page_of(a.block_table, a.max_pages, a.n_pages, b, (int)e);
      if (page >= 0) rid = page * CSA2_PAGE + (int)(e & (CSA2_PAGE - 1));
    }
    rowid[v] = rid;
  }
  __syncthreads();
  const int n_grp = (N + 15) >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int gpw = (n_grp + NW - 1) / NW;
  const int g0 = wv * gpw, g1 = min(n_grp, g0 + gpw);
  for (int r0 = g0; r0 < g1; r0 += kReindexRound) {
    u32x2 cd[kReindexRound];
    uint32_t sb[kReindexRound];
    int32_t rid[kReindexRound];
#pragma unroll
    for (int u = 0; u < kReindexRound; ++u) {
      const int v = (r0 + u) * 16 + n;
      rid[u] = (r0 + u < g1 && v < N) ? rowid[v] : -1;
    }
#pragma unroll
    for (int u = 0; u < kReindexRound; ++u) {
      cd[u] = u32x2{0u, 0u};
      sb[u] = 0u;
      if (rid[u] >= 0) {
        cd[u] = *reinterpret_cast<const u32x2*>(a.idx_codes + (int64_t)rid[u] * CSA2_IDX_CODE_BYTES + 8 * g);
        sb[u] = a.idx_scales[(int64_t)rid[u] * CSA2_IDX_SCALE_BYTES + (g >> 1)];
      }
    }
    // slot v's row id and key share a word; both are touched only by this wave,
    // in program order, so the read above precedes the write below
#pragma unroll
    for (int u = 0; u < kReindexRound; ++u) {
      if (r0 + u >= g1) break;                    // wave-uniform
      const float s = score16(cd[u], sb[u], a0, a1, wh);
      const int v = (r0 + u) * 16 + n;
      // validity lives in the lane that loaded the entry; lanes 0..15 hold g = 0
      if (lane < 16 && v < N) keys[v] = rid[u] >= 0 ? score_key(s) : 0u;
    }
  }
  __syncthreads();
  for (int i = N + threadIdx.x; i < kCap; i += kReindexThreads) keys[i] = 0u;
  __syncthreads();
  uint32_t kr[KPT];
  const int p0 = threadIdx.x * KPT;
#pragma unroll
  for (int i = 0; i < KPT; i += 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(keys + p0 + i);
    kr[i] = v.x;
    kr[i + 1] = v.y;
    kr[i + 2] = v.z;
    kr[i + 3] = v.w;
  }
  const SelectResult sr = block_select<kReindexThreads, KPT>(kr, a.topk, hist, scratch);
  int32_t* out = a.topk_idx + (int64_t)b * a.topk;
  block_emit<kReindexThreads, KPT>(kr, sr, scratch, [&](int i, uint32_t pos) {
    const int v = p0 + i;
    out[pos] = pool[v >> a.cb_shift] * cb + (v & (cb - 1));
  });
  for (int p = (int)sr.count + threadIdx.x; p < a.topk; p += kReindexThreads) out[p] = -1;
}


// Split Reindex, used when the caller passes a workspace.  One workgroup per sequence
// leaves all but B CUs idle while it gathers the pool's keys, and a single CU pulls
// scattered 272-byte pool blocks far slower than the GPU's bandwidth allows.  So the
// scoring runs over (sequence, 512-slot slice) workgroups that write key images to
// the workspace, and a second kernel selects the top-K of each sequence from them.
constexpr int kReSlice = 512;
constexpr int kReSelThreads = 1024;

__global__ __launch_bounds__(256) void reindex_score_kernel(ReindexArgs a, uint32_t* __restrict__ keys_ws) {
  const int b = blockIdx.x;
  const int cb = a.cand_block;
  const int N = a.pool_blocks * cb;
  const int v0 = blockIdx.y * kReSlice;
  if (v0 >= N) return;
  int64_t L = a.ctx_len[b];
  if (L < 0) L = 0;
  const int64_t n_vis = L >> a.vshift;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  bf16x8 a0, a1;
  load_q_frags(a.q_idx, b, a0, a1);
  float wh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) wh[h] = bf16_to_f32(a.w_idx[b * CSA2_H_INDEX + h]);
  const int32_t* pool = a.pool + (int64_t)b * a.pool_blocks;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  constexpr int kGroups = kReSlice / 16 / 4;    // 16-slot groups per wave
  // Slot of group u for this lane: v0 + (wid * kGroups + u) * 16 + n.  Three rounds of
  // loads (pool blocks, page ids, keys), each issued whole: lanes without a slot or an
  // entry load element 0 / row 0 (which exist whenever this workgroup runs) and drop
  // the value, so no branch splits a round and each round costs one wait.
  int blk[kGroups];
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const int v = v0 + (wid * kGroups + u) * 16 + n;
    const int bv = pool[v < N ? v >> a.cb_shift : 0];
    blk[u] = v < N ? bv : -1;
  }
  int pg[kGroups];
  int64_t ent[kGroups];
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const int v = v0 + (wid * kGroups + u) * 16 + n;
    ent[u] = (int64_t)blk[u] * cb + (v & (cb - 1));
    const bool ok = blk[u] >= 0 && ent[u] < n_vis && (ent[u] >> 6) < a.max_pages;
    const int p = bt[ok ? (int)(ent[u] >> 6) : 0];
    pg[u] = (ok && p >= 0 && p < a.n_pages) ? p : -1;
  }
  u32x2 cd[kGroups];
  uint32_t sb[kGroups];
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const int64_t row = pg[u] >= 0 ? (int64_t)pg[u] * CSA2_PAGE + (ent[u] & (CSA2_PAGE - 1)) : 0;
    const u32x2 cv = *reinterpret_cast<const u32x2*>(a.idx_codes + row * CSA2_IDX_CODE_BYTES + 8 * g);
    const uint32_t sv = a.idx_scales[row * CSA2_IDX_SCALE_BYTES + (g >> 1)];
    cd[u] = pg[u] >= 0 ? cv : u32x2{0u, 0u};
    sb[u] = pg[u] >= 0 ? sv : 0u;
  }
  uint32_t* kout = keys_ws + (int64_t)b * kReindexCap;
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const float s = score16(cd[u], sb[u], a0, a1, wh);
    const int v = v0 + (wid * kGroups + u) * 16 + n;
    if (lane < 16 && v < N) kout[v] = pg[u] >= 0 ? score_key(s) : 0u;
  }
}

template <int KPT>
__global__ __launch_bounds__(kReSelThreads) void reindex_select_kernel(ReindexArgs a, const uint32_t* __restrict__ keys_ws) {
  __shared__ __align__(16) uint32_t hist[kSelectHist];
  __shared__ uint32_t scratch[kSelectScratch];
  const int b = blockIdx.x;
  const int cb = a.cand_block;
  const int N = a.pool_blocks * cb;
  const int tid = threadIdx.x;
  const int p0 = tid * KPT;
  const int32_t* pool = a.pool + (int64_t)b * a.pool_blocks;
  // this thread's slots p0..p0+KPT-1 span at most two pool blocks (KPT <= 2 * cb or
  // the ids are re-read): fetch them before the select
  const int blo = p0 < N ? pool[p0 >> a.cb_shift] : -1;
  const int bhi = p0 + KPT - 1 < N ? pool[(p0 + KPT - 1) >> a.cb_shift] : -1;
  const uint32_t* kin = keys_ws + (int64_t)b * kReindexCap;
  uint32_t kr[KPT];
#pragma unroll
  for (int i = 0; i < KPT; i += 4) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (p0 + i < N) v = *reinterpret_cast<const u32x4*>(kin + p0 + i);
    kr[i] = p0 + i < N ? v.x : 0u;
    kr[i + 1] = p0 + i + 1 < N ? v.y : 0u;
    kr[i + 2] = p0 + i + 2 < N ? v.z : 0u;
    kr[i + 3] = p0 + i + 3 < N ? v.w : 0u;
  }
  const SelectResult sr = block_select<kReSelThreads, KPT>(kr, a.topk, hist, scratch);
  int32_t* out = a.topk_idx + (int64_t)b * a.topk;
  block_emit<kReSelThreads, KPT>(kr, sr, scratch, [&](int i, uint32_t pos) {
    const int v = p0 + i;
    const int bi = v >> a.cb_shift;
    const int blk = bi == (p0 >> a.cb_shift) ? blo : (bi == ((p0 + KPT - 1) >> a.cb_shift) ? bhi : pool[bi]);
    out[pos] = blk * cb + (v & (cb - 1));
  });
  for (int p = (int)sr.count + tid; p < a.topk; p += kReSelThreads) out[p] = -1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Kernels here take up to ~80 KB of dynamic LDS (gfx950 has 160 KB per CU); raise
// each kernel's limit once per process.
bool lds_limits_set() {
  static const bool ok = [] {
    const void* ks[] = {reinterpret_cast<const void*>(index_scan_kernel<4096, 1024>),
                        reinterpret_cast<const void*>(index_scan_kernel<4096>),
                        reinterpret_cast<const void*>(index_scan_kernel<8192>),
                        reinterpret_cast<const void*>(index_scan_kernel<16384>),
                        reinterpret_cast<const void*>(reindex_kernel<8>),
                        reinterpret_cast<const void*>(reindex_kernel<16>),
                        reinterpret_cast<const void*>(reindex_kernel<32>)};
    bool r = true;
    for (const void* k : ks)
      r = r && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess;
    return r;
  }();
  return ok;
}

}  // namespace

bool index_kernels_ready() { return lds_limits_set(); }

IndexFullPlan plan_index_full(int B, int64_t max_nvis, int topk, int pool_blocks, int cand_block) {
  IndexFullPlan p{};
  if (cand_block < 1) return p;
  int ch = 4096;
  while (ch < topk) ch *= 2;
  int64_t nc = (max_nvis + ch - 1) / ch;
  while (nc * topk > kMergeCap && ch < 16384) {
    ch *= 2;
    nc = (max_nvis + ch - 1) / ch;
  }
  if (nc < 1) nc = 1;
  if (nc * topk > kMergeCap || ch > 16384) return p;      // chunk = 0: unsupported
  // pool: the pool workgroup ranks at most kMergeCap block maxima of cand_block
  // entries (the only capacity check of the pool); their storage is sized for 1-entry
  // blocks, so the size does not depend on cand_block
  if (pool_blocks > 0 && (max_nvis + cand_block - 1) / cand_block > kMergeCap) return p;
  const int64_t max_blocks = pool_blocks > 0 ? std::max<int64_t>(max_nvis, 1) : 0;
  p.chunk = ch;
  p.n_chunks = (int)nc;
  p.max_blocks = (int)max_blocks;
  // group the chunks when the final merge would hold more than 16 keys per thread
  // (16 is faster than grouping for the mixed batch's longest sequences; 32 is not)
  const int64_t per_group = (4 * kMergeThreads) / topk;
  if (nc * topk > 16 * kMergeThreads && per_group >= 2) {
    p.group = (int)per_group;
    p.n_groups = (int)((nc + per_group - 1) / per_group);
  }
  size_t off = 0;
  p.off_cand_key = off;
  off = align256(off + (size_t)B * nc * topk * 4);
  p.off_cand_idx = off;
  off = align256(off + (size_t)B * nc * topk * 4);
  p.off_cand_cnt = off;
  off = align256(off + (size_t)B * nc * 4);
  p.off_blockmax = off;
  off = align256(off + (size_t)B * max_blocks * 4);
  p.off_grp_key = off;
  off = align256(off + (size_t)B * p.n_groups * topk * 4);
  p.off_grp_idx = off;
  off = align256(off + (size_t)B * p.n_groups * topk * 4);
  p.off_grp_cnt = off;
  off = align256(off + (size_t)B * p.n_groups * 4);
  p.total = off;
  return p;
}

namespace {

int index_full_impl(const csa2_cache_t& c, int B, const int32_t* ctx_len, int64_t max_ctx,
                    const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                    int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, const WriteArgs& wr,
                    hipStream_t s) {
  const int vs = vis_shift(c);
  const int64_t max_nvis = max_ctx >> vs;
  const IndexFullPlan p = plan_index_full(B, max_nvis, topk, pool_blocks, cand_block);
  if (p.chunk == 0) return CSA2_EUNSUPPORTED;
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
  sa.vshift = vs;
  sa.q_idx = q_idx;
  sa.w_idx = w_idx;
  sa.topk = topk;
  sa.n_chunks = p.n_chunks;
  sa.cand_block = cand_block;
  sa.want_blocks = pool_blocks > 0;
  sa.max_blocks = p.max_blocks;
  sa.cand_key = reinterpret_cast<uint32_t*>(w + p.off_cand_key);
  sa.cand_idx = reinterpret_cast<int32_t*>(w + p.off_cand_idx);
  sa.cand_cnt = reinterpret_cast<int32_t*>(w + p.off_cand_cnt);
  sa.block_max = reinterpret_cast<uint32_t*>(w + p.off_blockmax);
  sa.wr = wr;
  const size_t scan_lds = (size_t)(p.chunk + kSelectHist + kSelectScratch) * 4;
  const int64_t grid = (int64_t)B * p.n_chunks;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  if (p.chunk == 4096 && grid <= 256)
    hipLaunchKernelGGL((index_scan_kernel<4096, 1024>), dim3((unsigned)grid), dim3(1024), scan_lds, s, sa);
  else if (p.chunk == 4096)
    hipLaunchKernelGGL(index_scan_kernel<4096>, dim3((unsigned)grid), dim3(kScanThreads), scan_lds, s, sa);
  else if (p.chunk == 8192)
    hipLaunchKernelGGL(index_scan_kernel<8192>, dim3((unsigned)grid), dim3(kScanThreads), scan_lds, s, sa);
  else
    hipLaunchKernelGGL(index_scan_kernel<16384>, dim3((unsigned)grid), dim3(kScanThreads), scan_lds, s, sa);
  if (hip_status() != CSA2_OK) return CSA2_EHIP;

  MergeArgs ma;
  ma.ctx_len = ctx_len;
  ma.max_ctx = max_ctx;
  ma.vshift = vs;
  ma.topk = topk;
  ma.chunk = p.chunk;
  ma.n_chunks = p.n_chunks;
  if (p.group > 0) {
    GroupArgs ga;
    ga.ctx_len = ctx_len;
    ga.max_ctx = max_ctx;
    ga.vshift = vs;
    ga.topk = topk;
    ga.chunk = p.chunk;
    ga.n_chunks = p.n_chunks;
    ga.group = p.group;
    ga.n_groups = p.n_groups;
    ga.cand_key = sa.cand_key;
    ga.cand_idx = sa.cand_idx;
    ga.cand_cnt = sa.cand_cnt;
    ga.grp_key = reinterpret_cast<uint32_t*>(w + p.off_grp_key);
    ga.grp_idx = reinterpret_cast<int32_t*>(w + p.off_grp_idx);
    ga.grp_cnt = reinterpret_cast<int32_t*>(w + p.off_grp_cnt);
    hipLaunchKernelGGL(index_group_kernel<4>, dim3(B, p.n_groups), dim3(kMergeThreads), 0, s, ga);
    if (hip_status() != CSA2_OK) return CSA2_EHIP;
    ma.chunk = p.chunk * p.group;   // the final merge sees each group as one chunk
    ma.n_chunks = p.n_groups;
  }
  ma.cand_block = cand_block;
  ma.pool_blocks = pool_blocks;
  ma.max_blocks = p.max_blocks;
  ma.cand_key = p.group > 0 ? reinterpret_cast<uint32_t*>(w + p.off_grp_key) : sa.cand_key;
  ma.cand_idx = p.group > 0 ? reinterpret_cast<int32_t*>(w + p.off_grp_idx) : sa.cand_idx;
  ma.cand_cnt = p.group > 0 ? reinterpret_cast<int32_t*>(w + p.off_grp_cnt) : sa.cand_cnt;
  ma.block_max = sa.block_max;
  ma.topk_idx = topk_idx;
  ma.pool = pool;
  const int64_t n_cand = (int64_t)ma.n_chunks * topk;
  const int64_t n_blk = pool_blocks > 0 ? (max_nvis + cand_block - 1) / cand_block : 0;
  const int64_t need = n_cand > n_blk ? n_cand : n_blk;
  const dim3 mgrid(B, pool_blocks > 0 ? 2 : 1);
  if (need <= 4 * kMergeThreads)
    hipLaunchKernelGGL(index_merge_kernel<4>, mgrid, dim3(kMergeThreads), 0, s, ma);
  else if (need <= 8 * kMergeThreads)
    hipLaunchKernelGGL(index_merge_kernel<8>, mgrid, dim3(kMergeThreads), 0, s, ma);
  else if (need <= 16 * kMergeThreads)
    hipLaunchKernelGGL(index_merge_kernel<16>, mgrid, dim3(kMergeThreads), 0, s, ma);
  else
    hipLaunchKernelGGL(index_merge_kernel<32>, mgrid, dim3(kMergeThreads), 0, s, ma);
  return hip_status();
}

}  // namespace

int launch_index_full(const csa2_cache_t& c, int B, const int32_t* ctx_len, int64_t max_ctx,
                      const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                      int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, hipStream_t s) {
  WriteArgs none{};
  return index_full_impl(c, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks, cand_block, topk_idx, pool, ws,
                         none, s);
}

int launch_write_index_full(const csa2_cache_t& c, int B, const int32_t* start_tok, int T_new, const uint16_t* x,
                            const uint16_t* w, const uint16_t* k_idx, const int32_t* ctx_len, int64_t max_ctx,
                            const uint16_t* q_idx, const uint16_t* w_idx, int topk, int pool_blocks,
                            int cand_block, int32_t* topk_idx, int32_t* pool, void* ws, hipStream_t s) {
  const int ratio = cache_ratio(c);
  const int half = T_new / ratio;
  if (half > kScanMaxWrites) {
    // a wave stores its entries one after another, each a dependent round of loads:
    // past a decode step's few entries the write kernel's one wave per entry is faster
    const int rc = launch_write_kv(c, B, start_tok, T_new, x, w, k_idx, s);
    if (rc != CSA2_OK) return rc;
    return launch_index_full(c, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks, cand_block, topk_idx, pool,
                             ws, s);
  }
  const WriteArgs wr = write_args(c, start_tok, half, x, w, k_idx, ratio);
  return index_full_impl(c, B, ctx_len, max_ctx, q_idx, w_idx, topk, pool_blocks, cand_block, topk_idx, pool, ws,
                         wr, s);
}

size_t reindex_ws(int B) { return align256((size_t)B * kReindexCap * 4); }

int launch_reindex(const csa2_cache_t& c, int B, const int32_t* ctx_len, const uint16_t* q_idx,
                   const uint16_t* w_idx, const int32_t* pool, int pool_blocks, int cand_block,
                   int topk, int32_t* topk_idx, void* ws, size_t ws_bytes, hipStream_t s) {
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
  ra.vshift = vis_shift(c);
  ra.cb_shift = __builtin_ctz((unsigned)cand_block);   // cand_block: a power of two (checked at the boundary)
  const int N = pool_blocks * cand_block;
  if (ws && ws_bytes >= reindex_ws(B)) {
    uint32_t* keys = static_cast<uint32_t*>(ws);
    hipLaunchKernelGGL(reindex_score_kernel, dim3(B, (N + kReSlice - 1) / kReSlice), dim3(256), 0, s, ra, keys);
    if (hip_status() != CSA2_OK) return CSA2_EHIP;
    if (N <= 4 * kReSelThreads)
      hipLaunchKernelGGL(reindex_select_kernel<4>, dim3(B), dim3(kReSelThreads), 0, s, ra, keys);
    else if (N <= 8 * kReSelThreads)
      hipLaunchKernelGGL(reindex_select_kernel<8>, dim3(B), dim3(kReSelThreads), 0, s, ra, keys);
    else
      hipLaunchKernelGGL(reindex_select_kernel<16>, dim3(B), dim3(kReSelThreads), 0, s, ra, keys);
    return hip_status();
  }
  const int kpt = N <= 8 * kReindexThreads ? 8 : (N <= 16 * kReindexThreads ? 16 : 32);
  const size_t lds = (size_t)(kpt * kReindexThreads + kSelectHist + kSelectScratch) * 4;
  if (kpt == 8)
    hipLaunchKernelGGL(reindex_kernel<8>, dim3(B), dim3(kReindexThreads), lds, s, ra);
  else if (kpt == 16)
    hipLaunchKernelGGL(reindex_kernel<16>, dim3(B), dim3(kReindexThreads), lds, s, ra);
  else
    hipLaunchKernelGGL(reindex_kernel<32>, dim3(B), dim3(kReindexThreads), lds, s, ra);
  return hip_status();
}

}  // namespace csa2
