// Sparse gather-attention for launches with many (query, head group) pairs: the
// mixed serving batch and chunked prefill, where the work keeps every CU busy for
// several rounds and throughput, not the length of one workgroup's latency chain,
// sets the time.  Same computation as attention.hip (one softmax over the top-K FP4
// latent rows plus the bf16 window, K = V = the 512-d latent, fp32 accumulation,
// bf16 output); that file holds the kernel for small launches.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §1.2 (window 128,
// every head shares one 512-d latent) and §2.3.1 (each query attends to the selected
// entries and the layer's window KV together); [P3] "DeepSeek V4.1 Flash
// architecture..." (scores -> weights summing to 1 -> weighted sum of values).
//
// Two kernels:
//   sparse_decode_wide_kernel<G>  one workgroup (8 waves) per (query, 16G heads):
//                           G = 4 when H is a multiple of 64 and there are >= 512
//                           queries, else G = 2 when H is a multiple of 32.  Each
//                           row is read once per workgroup and each FP4 tile is
//                           converted once for G head groups;
//   sparse_decode_kernel<NW>  one workgroup of NW = 4 waves per (query, 16 heads)
//                           for the remaining head counts; at 81 KB of LDS two
//                           workgroups share a CU.
// Rows are processed in batches that live in one of two LDS buffers: window
// batches of bf16 rows (pitch 1040 B), then FP4 batches (256 code bytes + 16 scale
// bytes, pitch 272 B).  Batch k+1 is loaded when batch k starts -- the wide kernel
// copies it straight into the free buffer (global_load_lds), the 16-head kernel
// stages it in registers and stores it after batch k's PV -- so the loads overlap
// batch k's arithmetic.  Rows that are absent arrive as zeros, so stale bytes never
// meet a zero weight (0 * NaN is not 0).  The selected entries' page lookups
// are loads issued at the start and consumed only when the first FP4 batch is
// loaded, so they hide behind the window batches.  Per-wave timestamps on the
// MI355X (the mixed batch) put the time in each batch's vector ALU work and its
// three barriers, not in waiting for the next batch's rows, so the kernels keep
// vector instructions few: bf16 conversions in hardware, a chunk map without
// divisions, and window units that give every wave work.
// Per batch (16-head kernel):
//   QK  wave w scores 32-row tile w: D[row][head] via 16x16x32 bf16 MFMAs, A = rows
//       (lane: row l%16, dims 128g+8s..+7 at k-step s, g = l/16; FP4 rows become
//       bf16 through the hardware convert with the e8m0 scale folded in, exact),
//       B = q (lane: head l%16, same dims; q stays in registers).
//   max the batch maximum of every head goes through LDS, so all waves hold the
//       same running maximum, which is lazy (below).
//   P   the scoring wave turns its 32 scores per head into the P operand of the PV
//       MFMA -- a bf16 head plus a bf16 residual -- and parks it in LDS.  The lane's
//       scores are already the K-slots of that operand (rows 4g..4g+3 and
//       16+4g..16+4g+3 of head l%16), so no lane exchange is needed.
//   PV  every wave accumulates O[16 heads][its 64 dims] over all tiles of the batch:
//       n-tile t of lane column n is dim 64w + 4n + t, so a lane reads 4 adjacent
//       dims (2 FP4 bytes or 8 bf16 bytes) of each of its 8 rows and v_perm pairs
//       rows into the B operand.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kWaves = 8;             // the wide kernel
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = 272;           // FP4 row in LDS: 256 code bytes then 16 scale bytes
constexpr int kWinB = 1040;          // window row in LDS: 1024 bytes + 16 pad
constexpr int kPBytes = 32;          // per lane and tile: P head + residual

// Geometry of the 16-head kernel with NW waves: FP4 batches of 32*NW rows (one
// 32-row tile per wave), window batches of 8*NW rows, and 512/NW output dims per
// wave.  With 8 waves one workgroup fills a CU; with 4 waves a workgroup takes
// under half of the LDS, so two share a CU and each hides the other's loads.
template <int NW>
struct Geo16 {
  static constexpr int NT = NW * 64;
  static constexpr int FB = 32 * NW;                                  // FP4 rows per batch
  static constexpr int WB = 8 * NW;                                   // window rows per batch
  static constexpr int MT = NW;                                       // FP4 tiles per batch
  static constexpr int DW = CSA2_D_LATENT / NW;                       // output dims per wave
  static constexpr int NH = DW / 64;                                  // 64-dim accumulator groups
  static constexpr int BUF = FB * kRowB > WB * kWinB ? FB * kRowB : WB * kWinB;
  static constexpr int STAGE = (FB * 17 + NT - 1) / NT;              // 16-byte chunks per thread
  static constexpr int PSLOTS = MT + WB / 32;                         // FP4 tiles, then a window batch's
  static constexpr int OFF_P = 2 * BUF;                               // [PSLOTS][64 lanes][32 B]
  static constexpr int OFF_RID = OFF_P + PSLOTS * 64 * kPBytes;      // [2][FB] int32
  static constexpr int OFF_MAX = OFF_RID + 2 * FB * 4;               // [NW][16] float
  static constexpr int OFF_L = OFF_MAX + NW * 16 * 4;                // [NW][16] float
  static constexpr int LDS = OFF_L + NW * 16 * 4;
  // q of the 16 heads is staged at the window pitch in the P slots if they hold it,
  // else in buffer 1 (free until batch 1 is stored)
  static constexpr bool Q_IN_P = 16 * kWinB <= PSLOTS * 64 * kPBytes;
  static constexpr int OFF_Q = Q_IN_P ? OFF_P : BUF;
  static constexpr int QCH = 16 * CSA2_D_LATENT * 2 / 16 / NT;      // 16-byte q pieces per thread
  static_assert(WB * kWinB <= BUF && 16 * kWinB <= BUF, "window batch and q fit a buffer");
  static_assert(WB % 32 == 0 && (WB * 64) % NT == 0, "whole window tiles, whole chunks per thread");
  static_assert(NH >= 1 && NH * 64 * NW == CSA2_D_LATENT, "the waves split the dims in 64-dim groups");
  static_assert(2 * FB == NT, "one prefetched row id per thread (two FP4 batches)");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(NW == 8 || 2 * LDS <= 160 * 1024, "two 4-wave workgroups per CU");
};

constexpr float kLog2e = 1.4426950408889634f;
// The running maximum is lazy: it moves only when a batch's maximum passes it by more
// than 2^8 (weights up to 256 are exact in the bf16 head + residual split and in
// fp32 sums), so the accumulators are rarely rescaled.
constexpr float kLazy = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecArgs {
  const uint8_t* lat_codes;
  const uint8_t* lat_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* len;      // decode: context length; prefill: tokens before the chunk
  const uint16_t* q;
  const int32_t* topk_idx;
  int topk;
  const uint16_t* win;     // decode: ring [B][W][512]; prefill: [B][W-1+C][512]
  int W;
  float scale_log2;        // sm_scale * log2(e)
  uint16_t* out;
  float* lse;
  int vshift;              // token count -> visible entries: >> vshift
  int B, C, H, HG, prefill, q_per_xcd;
};

// low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

// Row of K-slot j for lane group g: rows 4g..4g+3, then 16+4g..16+4g+3.
__device__ __forceinline__ int slot_row(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// Window slot w (position t-W+1+w) holds a row, i.e. w < W and the position is >= 0.
__device__ __forceinline__ bool win_valid(int W, int t, int w) { return w < W && t - (W - 1) + w >= 0; }

// P operand (bf16 head + bf16 residual) of this lane's 8 scores (log2 units, -inf =
// absent) against the running max m; adds the weights to l_part.
__device__ __forceinline__ void make_p(const float (&z)[8], float m, float& l_part, u32x4& phi, u32x4& plo) {
  const float mb = (m == -INFINITY) ? 0.f : m;
  uint32_t h[4], r[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float p0 = __builtin_amdgcn_exp2f(z[j] - mb), p1 = __builtin_amdgcn_exp2f(z[j + 1] - mb);
    l_part += p0 + p1;
    split_pair(p0, p1, h[j >> 1], r[j >> 1]);
  }
  phi = u32x4{h[0], h[1], h[2], h[3]};
  plo = u32x4{r[0], r[1], r[2], r[3]};
}

// The same for the 4 scores of one 16-row half of a tile: half of the P operand.
__device__ __forceinline__ void make_p4(const float (&z)[4], float m, float& l_part, u32x2& phi, u32x2& plo) {
  const float mb = (m == -INFINITY) ? 0.f : m;
  uint32_t h[2], r[2];
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    const float p0 = __builtin_amdgcn_exp2f(z[j] - mb), p1 = __builtin_amdgcn_exp2f(z[j + 1] - mb);
    l_part += p0 + p1;
    split_pair(p0, p1, h[j >> 1], r[j >> 1]);
  }
  phi = u32x2{h[0], h[1]};
  plo = u32x2{r[0], r[1]};
}

// Scores of the FP4 tile at row `base` of the batch in LDS.
__device__ __forceinline__ void fp4_qk(const uint8_t* rows, const int32_t* rowid, int nrows, int base,
                                       const u32x4 (&qf)[16], float scale_log2, float (&z)[8]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  u32x4 cd0[4], cd1[4];
  const uint8_t* r0p = rows + (base + n) * kRowB;
  const uint8_t* r1p = rows + (base + 16 + n) * kRowB;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    cd0[c] = lds_ld<u32x4>(r0p + 64 * g + 16 * c);
    cd1[c] = lds_ld<u32x4>(r1p + 64 * g + 16 * c);
  }
  const uint32_t sb0 = lds_ld<uint32_t>(r0p + 256 + 4 * g);
  const uint32_t sb1 = lds_ld<uint32_t>(r1p + 256 + 4 * g);
  f32x4 sa[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float sc0 = e8m0_scale((sb0 >> (8 * c)) & 0xffu);
    const float sc1 = e8m0_scale((sb1 >> (8 * c)) & 0xffu);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, qf[4 * c + k]);
      const int e = k & 1;   // two partial sums per row half keep four MFMA chains in flight
      sa[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fp4x8_to_bf16x8(cd0[c][k], sc0)),
                                                      qv, sa[e], 0, 0, 0);
      sa[2 + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, fp4x8_to_bf16x8(cd1[c][k], sc1)), qv, sa[2 + e], 0, 0, 0);
    }
  }
  const f32x4 s0 = sa[0] + sa[1], s1 = sa[2] + sa[3];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r0 = base + slot_row(g, j), r1 = base + slot_row(g, 4 + j);
    z[j] = (r0 < nrows && rowid[r0] >= 0) ? s0[j] * scale_log2 : -INFINITY;
    z[4 + j] = (r1 < nrows && rowid[r1] >= 0) ? s1[j] * scale_log2 : -INFINITY;
  }
}

// Scores of the window tile at row `base` of the batch in LDS (window slots w0 + row).
__device__ __forceinline__ void win_qk(const uint8_t* wrows, int W, int t, int w0, int base, const u32x4 (&qf)[16],
                                       float scale_log2, float (&z)[8]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* r0p = wrows + (base + n) * kWinB + 256 * g;
  const uint8_t* r1p = wrows + (base + 16 + n) * kWinB + 256 * g;
  f32x4 sa[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 r0[8], r1[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r0[s] = lds_ld<u32x4>(r0p + 16 * (8 * half + s));
      r1[s] = lds_ld<u32x4>(r1p + 16 * (8 * half + s));
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, qf[8 * half + s]);
      const int e = s & 1;
      sa[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r0[s]), qv, sa[e], 0, 0, 0);
      sa[2 + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r1[s]), qv, sa[2 + e], 0, 0, 0);
    }
  }
  const f32x4 s0 = sa[0] + sa[1], s1 = sa[2] + sa[3];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z[j] = win_valid(W, t, w0 + base + slot_row(g, j)) ? s0[j] * scale_log2 : -INFINITY;
    z[4 + j] = win_valid(W, t, w0 + base + slot_row(g, 4 + j)) ? s1[j] * scale_log2 : -INFINITY;
  }
}

// Scores of the 16 window rows from row `base` of the batch in LDS (window slots
// w0 + row): lane (n, g) gets head n against rows base + 4g .. +3.
__device__ __forceinline__ void win_qk16(const uint8_t* wrows, int W, int t, int w0, int base,
                                         const u32x4 (&qf)[16], float scale_log2, float (&z)[4]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* rp = wrows + (base + n) * kWinB + 256 * g;
  f32x4 sa[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 rv[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) rv[s] = lds_ld<u32x4>(rp + 16 * (8 * half + s));
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sa[s & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rv[s]),
                                                          __builtin_bit_cast(bf16x8, qf[8 * half + s]), sa[s & 3], 0,
                                                          0, 0);
  }
  const f32x4 s = (sa[0] + sa[1]) + (sa[2] + sa[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = win_valid(W, t, w0 + base + 4 * g + j) ? s[j] * scale_log2 : -INFINITY;
}

// PV for this wave's 64 dims from 8 rows given as pairs d01[j] = dims (4n, 4n+1),
// d23[j] = dims (4n+2, 4n+3) of row slot j: n-tile t holds dim 4n + t.
__device__ __forceinline__ void pv4(f32x4 (&acc)[4], const uint32_t (&d01)[8], const uint32_t (&d23)[8], bf16x8 ph,
                                    bf16x8 pl) {
  bf16x8 bf[4];
  bf[0] = __builtin_bit_cast(bf16x8, u32x4{pack_lo(d01[0], d01[1]), pack_lo(d01[2], d01[3]),
                                           pack_lo(d01[4], d01[5]), pack_lo(d01[6], d01[7])});
  bf[1] = __builtin_bit_cast(bf16x8, u32x4{pack_hi(d01[0], d01[1]), pack_hi(d01[2], d01[3]),
                                           pack_hi(d01[4], d01[5]), pack_hi(d01[6], d01[7])});
  bf[2] = __builtin_bit_cast(bf16x8, u32x4{pack_lo(d23[0], d23[1]), pack_lo(d23[2], d23[3]),
                                           pack_lo(d23[4], d23[5]), pack_lo(d23[6], d23[7])});
  bf[3] = __builtin_bit_cast(bf16x8, u32x4{pack_hi(d23[0], d23[1]), pack_hi(d23[2], d23[3]),
                                           pack_hi(d23[4], d23[5]), pack_hi(d23[6], d23[7])});
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bf[t], acc[t], 0, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bf[t], acc[t], 0, 0, 0);
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 8 / NW) void sparse_decode_kernel(DecArgs a) {
  using G = Geo16<NW>;
  constexpr int NT = G::NT, FB = G::FB, WB = G::WB, STAGE = G::STAGE, BUF = G::BUF, NH = G::NH;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* plds = lds + G::OFF_P;
  int32_t* rowid_all = reinterpret_cast<int32_t*>(lds + G::OFF_RID);
  float* m_part = reinterpret_cast<float*>(lds + G::OFF_MAX);
  float* l_w = reinterpret_cast<float*>(lds + G::OFF_L);

  // XCD-aware mapping: consecutive workgroup ids go to different XCDs; XCD x takes
  // the contiguous query range [x * q_per_xcd, (x+1) * q_per_xcd), all head groups.
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int ql = li / a.HG;
  const int hg = li - ql * a.HG;
  const int64_t qi = (int64_t)xcd * a.q_per_xcd + ql;
  if (ql >= a.q_per_xcd || qi >= (int64_t)a.B * a.C) return;
  const int b = (int)(qi / a.C);
  const int ci = (int)(qi - (int64_t)b * a.C);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;

  // the workgroup's rows: window rows [wr0, wr1), FP4 rows [fr0, fr1) of topk_idx
  const int wr0 = 0, wr1 = a.W, fr0 = 0, fr1 = a.topk;

  int64_t Lq = a.len[b];
  if (Lq < 0) Lq = 0;
  if (a.prefill) Lq += ci + 1;   // chunk query ci sits at position prior + ci
  const int n_vis = (int)(Lq >> a.vshift);
  const int t = (int)Lq - 1;
  const uint16_t* win_b = a.win + (int64_t)b * (a.prefill ? a.W - 1 + a.C : a.W) * CSA2_D_LATENT;
  const int32_t* tk = a.topk_idx + qi * a.topk;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  const int n_wb = (wr1 - wr0 + WB - 1) / WB;
  const int n_fb = (fr1 - fr0 + FB - 1) / FB;
  const int nb = n_wb + n_fb;

  // row id of entry e (-1: invalid id, absent page)
  auto row_of = [&](int e, int page) -> int {
    return (e >= 0 && e < n_vis && page >= 0 && page < a.n_pages) ? page * CSA2_PAGE + (e & (CSA2_PAGE - 1)) : -1;
  };
  auto page_ok = [&](int e) { return e >= 0 && e < n_vis && (e >> 6) < a.max_pages; };
  // FP4 batch f >= 2: ids resolved when the batch is issued
  auto resolve_rows = [&](int f) {
    const int r0 = fr0 + f * FB;
    const int nrows = min(fr1 - r0, FB);
    int32_t* rowid = rowid_all + (f & 1) * FB;
    for (int i = tid; i < FB; i += NT) {
      const int e = i < nrows ? tk[r0 + i] : -1;
      rowid[i] = page_ok(e) ? row_of(e, bt[e >> 6]) : -1;
    }
  };
  // Batch k in registers: thread tid holds chunks c = tid + 512u (16 bytes each) of
  // the batch image -- FP4: piece c%17 of row c/17 (16 code pieces, then the scales);
  // window: piece c%64 of row c/64 -- zeros where no row is.  Every chunk is loaded
  // (one with no row reads window row 0 of the sequence or cache row 0, and is
  // dropped), so no branch splits the loads: they issue back to back.
  auto load_batch = [&](int k, u32x4 (&st)[STAGE]) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (k < n_wb) {
      const int w0 = wr0 + k * WB;
      int slot0 = (t - (a.W - 1) + w0) % a.W;   // ring slot of the batch's first position
      if (slot0 < 0) slot0 += a.W;
#pragma unroll
      for (int u = 0; u < WB * 64 / NT; ++u) {
        const int c = tid + NT * u;
        const int r = c >> 6, piece = c & 63;
        const bool ok = w0 + r < wr1 && win_valid(a.W, t, w0 + r);
        int row = a.prefill ? ci + w0 + r : (slot0 + r >= a.W ? slot0 + r - a.W : slot0 + r);
        row = ok ? row : 0;
        const u32x4 v = *reinterpret_cast<const u32x4*>(win_b + (int64_t)row * CSA2_D_LATENT + 8 * piece);
        st[u] = ok ? v : zero;
      }
#pragma unroll
      for (int u = WB * 64 / NT; u < STAGE; ++u) st[u] = zero;
    } else {
      const int f = k - n_wb;
      const int nrows = min(fr1 - fr0 - f * FB, FB);
      const int32_t* rowid = rowid_all + (f & 1) * FB;
      int rid[STAGE];
#pragma unroll
      for (int u = 0; u < STAGE; ++u) {
        const int c = tid + NT * u;
        rid[u] = rowid[min(c / 17, FB - 1)];
      }
#pragma unroll
      for (int u = 0; u < STAGE; ++u) {
        const int c = tid + NT * u;
        const int r = c / 17, piece = c - r * 17;
        const bool ok = c < FB * 17 && r < nrows && rid[u] >= 0;
        const int64_t rw = ok ? rid[u] : 0;
        const uint8_t* src = piece < 16 ? a.lat_codes + rw * CSA2_LAT_CODE_BYTES + 16 * piece
                                        : a.lat_scales + rw * CSA2_LAT_SCALE_BYTES;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        st[u] = ok ? v : zero;
      }
    }
  };
  auto store_batch = [&](int k, const u32x4 (&st)[STAGE]) {
    uint8_t* buf = lds + (k & 1) * BUF;
    if (k < n_wb) {
#pragma unroll
      for (int u = 0; u < WB * 64 / NT; ++u) {
        const int c = tid + NT * u;
        *reinterpret_cast<u32x4*>(buf + (c >> 6) * kWinB + (c & 63) * 16) = st[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < STAGE; ++u) {
        const int c = tid + NT * u;
        if (c < FB * 17) *reinterpret_cast<u32x4*>(buf + c * 16) = st[u];
      }
    }
  };

  // ---- start: the entry ids of the first two FP4 batches (thread tid: batch tid/256,
  // row tid%256) go out first, then batch 0 (window rows need no lookups) and q.  The
  // ids' page lookups are issued as soon as the ids land, while the rest is in flight.
  u32x4 st[STAGE];
  const int pf_i = tid % FB, pf_f = tid / FB;
  const int pf_r = fr0 + pf_f * FB + pf_i;
  const int pf_e = (pf_f < n_fb && pf_r < fr1) ? tk[pf_r] : -1;
  // q of the 16 heads is read from memory once per workgroup -- thread tid: head
  // tid/TPH, QCH 16-byte pieces from dim 8*QCH*(tid%TPH) -- and handed to the waves
  // through LDS at the window pitch, as win_qk reads rows: in the P slots, free until
  // the first P, or in buffer 1, free until batch 1 is stored.
  constexpr int TPH = NT / 16;   // threads per head
  u32x4 qs[G::QCH];
  {
    const uint16_t* qp = a.q + (qi * a.H + hg * 16 + tid / TPH) * CSA2_D_LATENT + 8 * G::QCH * (tid % TPH);
#pragma unroll
    for (int u = 0; u < G::QCH; ++u) qs[u] = *reinterpret_cast<const u32x4*>(qp + 8 * u);
  }
  // W >= 1 (checked by the launcher), so the run starts with a window batch, which
  // needs no lookups; the ids' page lookups are issued behind it.
  load_batch(0, st);
  int pf_page = -1;
  if (page_ok(pf_e)) pf_page = bt[pf_e >> 6];
  store_batch(0, st);
  // q and the entry ids have arrived before the loop starts: the wait counts inside
  // the loop then cover only the next batch's loads, which stay in flight until the
  // batch is stored after PV.
  __builtin_amdgcn_s_waitcnt(0);
  {
    uint8_t* qd = lds + G::OFF_Q + (tid / TPH) * kWinB + 16 * G::QCH * (tid % TPH);
#pragma unroll
    for (int u = 0; u < G::QCH; ++u) *reinterpret_cast<u32x4*>(qd + 16 * u) = qs[u];
  }
  u32x4 qf[16];   // q operand of head hg*16+n: dims 128g + 8s .. +7 for k-step s
  auto read_q = [&]() {   // after a barrier that follows the stores above
    const uint8_t* qp = lds + G::OFF_Q + n * kWinB + 256 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = lds_ld<u32x4>(qp + 16 * s);
  };

  f32x4 acc[NH][4];   // group hh: dims DW*wid + 64*hh .. +63
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[hh][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY, l_part = 0.f;

  // PV of one 32-row tile of a batch in LDS (window rows: bf16; else FP4), this wave's
  // DW dims, with the P operand from P slot ps.
  auto pv_tile = [&](const uint8_t* buf, bool win, int tile, int ps) {
    const uint8_t* pp = plds + (ps * 64 + lane) * kPBytes;
    const bf16x8 ph = __builtin_bit_cast(bf16x8, lds_ld<u32x4>(pp));
    const bf16x8 pl = __builtin_bit_cast(bf16x8, lds_ld<u32x4>(pp + 16));
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      const int d0 = G::DW * wid + 64 * hh;   // first dim of the group
      uint32_t d01[8], d23[8];
      if (win) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2 v = lds_ld<u32x2>(buf + (tile * 32 + slot_row(g, j)) * kWinB + 2 * d0 + 8 * n);
          d01[j] = v.x;
          d23[j] = v.y;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint8_t* rp = buf + (tile * 32 + slot_row(g, j)) * kRowB;
          const uint32_t c2 = lds_ld<uint16_t>(rp + d0 / 2 + 2 * n);
          const float sc = e8m0_scale(rp[256 + d0 / 32 + (n >> 3)]);
          d01[j] = fp4x2_to_bf16x2<0>(c2, sc);
          d23[j] = fp4x2_to_bf16x2<1>(c2, sc);
        }
      }
      pv4(acc[hh], d01, d23, ph, pl);
    }
  };
  auto put_p = [&](const float (&z)[8], float m, int ps) {
    u32x4 ph, pl;
    make_p(z, m, l_part, ph, pl);
    uint8_t* pp = plds + (ps * 64 + lane) * kPBytes;
    *reinterpret_cast<u32x4*>(pp) = ph;
    *reinterpret_cast<u32x4*>(pp + 16) = pl;
  };

  if (n_wb == 1 && n_fb == 1) {
    // One window batch (buffer 0, stored in the prologue) and one FP4 batch (buffer 1)
    // in a single pass: the window tiles are scored while the FP4 rows load, then one
    // softmax and one PV cover all tiles.
    uint8_t* bufw = lds;
    uint8_t* buff = lds + BUF;
    const int ntl_w = (min(wr1 - wr0, WB) + 31) >> 5;
    const int nrows_f = min(fr1 - fr0, FB);
    const int ntl_f = (nrows_f + 31) >> 5;
    rowid_all[tid] = row_of(pf_e, pf_page);
    __syncthreads();   // window rows, q and the FP4 row ids stored by every thread
    load_batch(1, st);   // FP4 rows: in flight while the window tiles are scored
    read_q();
    float zw[8], zf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) zw[j] = zf[j] = -INFINITY;
    if (wid < ntl_w) win_qk(bufw, a.W, t, wr0, wid * 32, qf, a.scale_log2, zw);
    if constexpr (!G::Q_IN_P) __syncthreads();   // q, staged in buffer 1, read by every wave
    store_batch(1, st);
    __syncthreads();   // FP4 rows stored by every thread
    if (wid < ntl_f) fp4_qk(buff, rowid_all, nrows_f, wid * 32, qf, a.scale_log2, zf);
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) tmax = fmaxf(tmax, fmaxf(zw[j], zf[j]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    if (g == 0) m_part[wid * 16 + n] = tmax;
    __syncthreads();
    float mb = m_part[n];
#pragma unroll
    for (int w = 1; w < NW; ++w) mb = fmaxf(mb, m_part[w * 16 + n]);
    if (wid < ntl_f) put_p(zf, mb, wid);
    if (wid < ntl_w) put_p(zw, mb, G::MT + wid);
    m_run = mb;
    __syncthreads();
#pragma unroll 1
    for (int tile = 0; tile < ntl_w; ++tile) pv_tile(bufw, true, tile, G::MT + tile);
#pragma unroll 1
    for (int tile = 0; tile < ntl_f; ++tile) pv_tile(buff, false, tile, tile);
  } else {
  __syncthreads();   // q stored by every thread
  read_q();
#pragma unroll 1
  for (int k = 0; k < nb; ++k) {
    const bool is_win = k < n_wb;
    uint8_t* buf = lds + (k & 1) * BUF;
    const int f = k - n_wb;
    const int w0 = wr0 + k * WB;
    const int nrows = is_win ? min(wr1 - w0, WB) : min(fr1 - fr0 - f * FB, FB);
    const int32_t* rowid = rowid_all + (f & 1) * FB;
    const int ntl = (nrows + 31) >> 5;

    __syncthreads();   // batch k stored by every thread; batch k-1 fully consumed
    // Batch k+1 is loaded now if its rows are known (a window batch, or the second FP4
    // batch whose ids came with the first); otherwise its row ids are resolved after
    // this batch's QK, which hides the lookups, and it is loaded after the next barrier.
    const int f1 = k + 1 - n_wb;
    const bool has_next = k + 1 < nb;
    const bool ids_later = has_next && (f1 == 0 || f1 >= 2);
    if (has_next && !ids_later) load_batch(k + 1, st);   // stored after this batch's PV

    // ---- QK: wave w scores tile w ----
    float z[8];
    if (wid < ntl) {
      if (is_win)
        win_qk(buf, a.W, t, w0, wid * 32, qf, a.scale_log2, z);
      else
        fp4_qk(buf, rowid, nrows, wid * 32, qf, a.scale_log2, z);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) z[j] = -INFINITY;
    }
    float tmax = z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, z[j]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    if (g == 0) m_part[wid * 16 + n] = tmax;
    if (ids_later) {
      if (f1 == 0)
        rowid_all[tid] = row_of(pf_e, pf_page);   // the two prefetched FP4 batches
      else
        resolve_rows(f1);
    }
    __syncthreads();
    if (ids_later) load_batch(k + 1, st);

    // ---- batch max of head n (identical in every wave), P for the scored tile ----
    float mb = m_part[n];
#pragma unroll
    for (int w = 1; w < NW; ++w) mb = fmaxf(mb, m_part[w * 16 + n]);
    const float m_new = mb > m_run + kLazy ? mb : m_run;   // lazy: moves only past 2^8 headroom
    const float fac = (m_run == -INFINITY || m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_part *= fac;
    if (wid < ntl) put_p(z, m_new, wid);
    // rescale: acc[t][i] belongs to head 4g+i, whose factor lives in lane 4g+i
    {
      float fo[4];
      bool any = false;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        fo[ii] = __shfl(fac, 4 * g + ii, kWave);
        any = any || fo[ii] != 1.f;
      }
      if (__any(any)) {
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[hh][tt][ii] *= fo[ii];
          }
        }
      }
    }
    m_run = m_new;
    __syncthreads();

    // ---- PV over every tile of the batch, this wave's 64 dims ----
#pragma unroll 1
    for (int tile = 0; tile < ntl; ++tile) pv_tile(buf, is_win, tile, tile);
    if (k + 1 < nb) store_batch(k + 1, st);   // into the other buffer, free since batch k began
  }
  }

  // ---- softmax denominators, output ----
  float l_head = l_part;
  l_head += __shfl_xor(l_head, 16, kWave);
  l_head += __shfl_xor(l_head, 32, kWave);
  if (g == 0) l_w[wid * 16 + n] = l_head;
  __syncthreads();
  float lh[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += l_w[w * 16 + 4 * g + ii];
    lh[ii] = s;
  }
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const float inv = lh[ii] > 0.f ? __builtin_amdgcn_rcpf(lh[ii]) : 0.f;
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      *reinterpret_cast<u32x2*>(a.out + (qi * a.H + hg * 16 + 4 * g + ii) * CSA2_D_LATENT + G::DW * wid + 64 * hh +
                                4 * n) = u32x2{pack_bf16x2(acc[hh][0][ii] * inv, acc[hh][1][ii] * inv),
                                               pack_bf16x2(acc[hh][2][ii] * inv, acc[hh][3][ii] * inv)};
    }
  }
  if (a.lse && wid == 0 && g == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += l_w[w * 16 + n];
    a.lse[qi * a.H + hg * 16 + n] = s > 0.f ? (m_run + log2f(s)) * kLn2 : -INFINITY;
  }
}


// ---------------------------------------------------------------------------------
// 16G heads of a query in one workgroup (G = 2 or 4).  The 16-head kernel above
// converts every FP4 element once per head group; here the PV operand of a row is
// converted once and feeds the MFMAs of all G head groups, and every row is read
// from memory once per workgroup instead of once per head group.
//   batches  window batches of 64 rows and FP4 batches of 128 rows, double-
//            buffered, copied straight into LDS: a window row is one 1 KB copy, an
//            FP4 batch image (17 16-byte pieces per row) 34 copies of 1 KB.  With no
//            staging registers the 64-head instance fits 64-row window batches too
//            (two barriers' worth of fixed cost fewer than four 32-row batches).
//   QK       FP4 unit (tile t, head group h) = the scores of 16 heads x 32 rows;
//            wave w takes head group w%G (its q fragments stay in registers) and
//            tile w/G (G = 2), or tiles w/4 and w/4 + 2 (G = 4).  Window unit
//            (tile w/4, head group, and with G = 2 a 16-row half): one per wave.
//   max, P   per head group through LDS, as above; P of every unit is parked in LDS
//            (a window half fills half of its tile's P operand), an FP4 batch's in
//            the unused tail of its own buffer.
//   PV       wave w accumulates O[16G heads][dims 64w..64w+63] (16G registers): per
//            tile it converts its 8 rows x 4 dims once and runs the 2 x 4 MFMAs of
//            each head group on them.
// ---------------------------------------------------------------------------------
constexpr int64_t kH64MinQueries = 512;                   // launches with fewer queries use 32 heads
constexpr int kFb64 = 128;                                // FP4 rows per batch (4 tiles)
constexpr int kTiles64 = kFb64 / 32;
constexpr int kPf64 = 4;                                  // FP4 batches whose ids are prefetched
static_assert(kPf64 * kFb64 == kThreads, "one prefetched row id per thread");

// Geometry of the kernel with G head groups.  Batches are copied from memory straight
// into LDS (global_load_lds), so a batch in flight holds no registers.  A window batch
// is 64 rows (two tiles); its units (tile, head group, and with G = 2 a 16-row half)
// give every wave one.  An FP4 batch is 128 rows; its P operands sit in the unused
// tail of its own buffer, the window batches' in an area of their own.
template <int G>
struct GeoW {
  static constexpr int WB = 64;                                        // window rows per batch
  static constexpr int PF = kTiles64 * G * 64 * kPBytes;               // P of an FP4 batch
  static constexpr int BUF = WB * kWinB > kFb64 * kRowB + PF ? WB * kWinB : kFb64 * kRowB + PF;
  static constexpr int OFF_PF = kFb64 * kRowB;                          // in the FP4 batch's buffer
  static constexpr int OFF_PW = 2 * BUF;                                // [2 tiles][G groups][64 lanes][32 B]
  static constexpr int OFF_RID = OFF_PW + (WB / 32) * G * 64 * kPBytes; // [4][128] int32
  static constexpr int OFF_MAX = OFF_RID + kPf64 * kFb64 * 4;          // [8 waves][16] float
  static constexpr int OFF_L = OFF_MAX + kWaves * 16 * 4;              // [8 waves][16] float
  static constexpr int LDS = OFF_L + kWaves * 16 * 4;
  static_assert(WB / 32 * G * (G == 2 ? 2 : 1) == kWaves, "one window unit per wave");
  static_assert(WB % kWaves == 0, "whole window rows per wave");
  static_assert(kTiles64 * G * 2 >= kWaves && kTiles64 * G % kWaves == 0, "whole FP4 units per wave");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};
constexpr int kFpDma = kFb64 * 17 / 64;     // 1 KB copies of an FP4 batch image (34)
static_assert(kFb64 * 17 % 64 == 0 && kFpDma > 4 * kWaves && kFpDma <= 5 * kWaves, "4 or 5 copies per wave");

// Rows that are absent (window slots before position 0, invalid ids, unmapped pages,
// the tail of the last batch) are copied from here, so stale LDS bytes never meet a
// zero weight (0 * NaN is not 0).  Read only; zero from load time.
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[1024];

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// 16 bytes per lane from global memory into LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
}
__device__ __forceinline__ void wait_all_vm() { __builtin_amdgcn_s_waitcnt(0x3f70); }   // vmcnt(0)
// Workgroup barrier after this wave's LDS accesses have completed.  Bare: the fence of
// __syncthreads would also wait for the LDS copies in flight.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

template <int G>
__global__ __launch_bounds__(kThreads) void sparse_decode_wide_kernel(DecArgs a) {
  static_assert(G == 2 || G == 4, "32 or 64 heads per workgroup");
  constexpr int WPG = kWaves / G;                // waves per head group
  using GW = GeoW<G>;
  constexpr int WB = GW::WB;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int32_t* rowid_all = reinterpret_cast<int32_t*>(lds + GW::OFF_RID);
  float* m_part = reinterpret_cast<float*>(lds + GW::OFF_MAX);
  float* l_w = reinterpret_cast<float*>(lds + GW::OFF_L);

  // XCD-aware mapping: XCD x takes the contiguous query range [x * q_per_xcd, ...).
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int nhq = a.H / (16 * G);               // workgroups per query
  const int ql = li / nhq;
  const int hq = li - ql * nhq;                 // heads 16G*hq .. +16G-1
  const int64_t qi = (int64_t)xcd * a.q_per_xcd + ql;
  if (ql >= a.q_per_xcd || qi >= (int64_t)a.B * a.C) return;
  const int b = (int)(qi / a.C);
  const int ci = (int)(qi - (int64_t)b * a.C);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int my_hg = wid % G;                    // head group of this wave's QK units

  int64_t Lq = a.len[b];
  if (Lq < 0) Lq = 0;
  if (a.prefill) Lq += ci + 1;
  const int n_vis = (int)(Lq >> a.vshift);
  const int t = (int)Lq - 1;
  const uint16_t* win_b = a.win + (int64_t)b * (a.prefill ? a.W - 1 + a.C : a.W) * CSA2_D_LATENT;
  const int32_t* tk = a.topk_idx + qi * a.topk;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  const int n_wb = (a.W + WB - 1) / WB;
  const int n_fb = a.topk > 0 ? (a.topk + kFb64 - 1) / kFb64 : 0;
  const int nb = n_wb + n_fb;

  auto row_of = [&](int e, int page) -> int {
    return (e >= 0 && e < n_vis && page >= 0 && page < a.n_pages) ? page * CSA2_PAGE + (e & (CSA2_PAGE - 1)) : -1;
  };
  auto page_ok = [&](int e) { return e >= 0 && e < n_vis && (e >> 6) < a.max_pages; };
  auto resolve_rows = [&](int f) {   // FP4 batch f >= kPf64, into slot f % kPf64
    const int r0 = f * kFb64;
    const int nrows = min(a.topk - r0, kFb64);
    int32_t* rowid = rowid_all + (f % kPf64) * kFb64;
    for (int i = tid; i < kFb64; i += kThreads) {
      const int e = i < nrows ? tk[r0 + i] : -1;
      rowid[i] = page_ok(e) ? row_of(e, bt[e >> 6]) : -1;
    }
  };
  // Batch j into buffer j % 2.  Window: wave w copies rows w + 8u, one 1 KB copy per
  // row at the padded pitch.  FP4: 1 KB copy c of the batch image (chunk 64c + lane
  // is piece p of row r, 17 pieces per row: 16 of codes, then the scales) for
  // c = w + 8u.
  const uint8_t* zero = g_zero_row;
  int rp_pk[5];   // FP4 copy u of this lane: row r and piece p of chunk 64c + lane, as (r << 5) | p
#pragma unroll
  for (int u = 0; u < 5; ++u) {
    const int ch = 64 * (wid + kWaves * u) + lane;
    const int r = ch / 17;
    rp_pk[u] = (r << 5) | (ch - 17 * r);
  }
  auto issue_batch = [&](int j) __attribute__((always_inline)) {
    uint8_t* buf = lds + (j & 1) * GW::BUF;
    if (j < n_wb) {
      const int w0 = j * WB;
#pragma unroll
      for (int u = 0; u < WB / kWaves; ++u) {
        const int r = wid + kWaves * u;
        const int sl = w0 + r;                     // window slot: position t - (W-1) + sl
        const uint8_t* src = zero + 16 * lane;
        if (win_valid(a.W, t, sl)) {
          int row;
          if (a.prefill) {
            row = ci + sl;
          } else {
            row = (t - (a.W - 1) + sl) % a.W;
            row = row < 0 ? row + a.W : row;
          }
          src = reinterpret_cast<const uint8_t*>(win_b + (int64_t)row * CSA2_D_LATENT) + 16 * lane;
        }
        dma16(src, buf + r * kWinB);
      }
    } else {
      const int f = j - n_wb;
      const int nrows = min(a.topk - f * kFb64, kFb64);
      const int32_t* rowid = rowid_all + (f % kPf64) * kFb64;
#pragma unroll
      for (int u = 0; u < 5; ++u) {
        const int c = wid + kWaves * u;
        if (c < kFpDma) {
          const int r = rp_pk[u] >> 5, p = rp_pk[u] & 31;
          const int rid = r < nrows ? rowid[r] : -1;
          // one 64-bit add per copy in the loop: hoisted per-copy pointers would hold
          // registers across the whole batch loop
          const uint8_t* base = rid < 0 ? zero : (p < 16 ? a.lat_codes : a.lat_scales);
          const uint64_t off = rid < 0 ? (uint64_t)(16 * p)
                                       : (p < 16 ? ((uint64_t)rid << 8) + (uint64_t)(16 * p) : (uint64_t)rid << 4);
          dma16(base + off, buf + 1024 * c);
        }
      }
    }
  };

  // ---- start ----
  const int pf_f = tid / kFb64, pf_r = tid;     // prefetched id: FP4 batch tid/128, row tid%128
  const int pf_e = (pf_f < n_fb && pf_r < a.topk) ? tk[pf_r] : -1;
  u32x4 qf[16];   // q operand of head 16G*hq + 16*my_hg + n: dims 128g + 8s .. +7
  {
    const uint16_t* qp = a.q + (qi * a.H + 16 * G * hq + 16 * my_hg + n) * CSA2_D_LATENT + 128 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qp + 8 * s);
  }
  int pf_page = -1;
  if (n_wb > 0) issue_batch(0);
  wait_all_vm();

  f32x4 acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[h][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[G];   // head n of group h
#pragma unroll
  for (int h = 0; h < G; ++h) m_run[h] = -INFINITY;
  float l_part = 0.f;                                                 // head n of my_hg

#pragma unroll 1
  for (int k = 0; k < nb; ++k) {
    const bool is_win = k < n_wb;
    uint8_t* buf = lds + (k & 1) * GW::BUF;
    const int f = k - n_wb;
    const int w0 = k * WB;
    const int nrows = is_win ? min(a.W - w0, WB) : min(a.topk - f * kFb64, kFb64);
    const int32_t* rowid = rowid_all + (f % kPf64) * kFb64;
    const int ntl = (nrows + 31) >> 5;

    uint8_t* plds = is_win ? lds + GW::OFF_PW : buf + GW::OFF_PF;   // P of this batch's units
    barrier_lds();   // batch k copied in by every wave; batch k-1 fully consumed
    if (k == 0 && page_ok(pf_e)) pf_page = bt[pf_e >> 6];
    if (k + 1 < nb) {
      const int f1 = k + 1 - n_wb;
      if (f1 == 0) {
        rowid_all[tid] = row_of(pf_e, pf_page);
        barrier_lds();
      } else if (f1 >= kPf64) {
        resolve_rows(f1);
        barrier_lds();
      }
      issue_batch(k + 1);   // into the other buffer, free since batch k began
    }

    // ---- QK.  FP4: units (tile w/G, group w%G) and, with 4 groups, (tile w/4 + 2,
    // group w%4).  Window: unit (tile wt = w/4, group w%G), with 2 groups only rows
    // 16wq .. +15 of the tile. ----
    const int t0 = wid / G, t1 = t0 + 2;
    const int wt = wid / 4, wq = (wid / G) & 1;
    float z0[8], z1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) z0[j] = z1[j] = -INFINITY;
    if (is_win) {
      if (wt < ntl) {
        if constexpr (G == 2) {
          float zh[4];
          win_qk16(buf, a.W, t, w0, 32 * wt + 16 * wq, qf, a.scale_log2, zh);
#pragma unroll
          for (int j = 0; j < 4; ++j) z0[j] = zh[j];
        } else {
          win_qk(buf, a.W, t, w0, 32 * wt, qf, a.scale_log2, z0);
        }
      }
    } else {
      if (t0 < ntl) fp4_qk(buf, rowid, nrows, t0 * 32, qf, a.scale_log2, z0);
      if (G == 4 && t1 < ntl) fp4_qk(buf, rowid, nrows, t1 * 32, qf, a.scale_log2, z1);
    }
    float tmax = z0[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) tmax = fmaxf(tmax, fmaxf(z0[j], z1[j]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    if (g == 0) m_part[wid * 16 + n] = tmax;

    // ---- P of this wave's units against its group's running maximum, written before
    // the barrier.  It stands unless some group's maximum moves, which the lazy
    // maximum makes rare after the first rows: then it is written again. ----
    float my_m = m_run[0];
#pragma unroll
    for (int h = 1; h < G; ++h) my_m = my_hg == h ? m_run[h] : my_m;
    auto write_p = [&](float mref) -> float {
      float l_add = 0.f;
      if (is_win) {
        if (wt < ntl) {
          if constexpr (G == 2) {
            // K-slots 4wq .. 4wq+3 of the tile's P operand: rows 16wq + 4g .. +3
            const float zh[4] = {z0[0], z0[1], z0[2], z0[3]};
            u32x2 ph, pl;
            make_p4(zh, mref, l_add, ph, pl);
            uint8_t* pp = plds + ((wt * G + my_hg) * 64 + lane) * kPBytes + 8 * wq;
            *reinterpret_cast<u32x2*>(pp) = ph;
            *reinterpret_cast<u32x2*>(pp + 16) = pl;
          } else {
            u32x4 ph, pl;
            make_p(z0, mref, l_add, ph, pl);
            uint8_t* pp = plds + ((wt * G + my_hg) * 64 + lane) * kPBytes;
            *reinterpret_cast<u32x4*>(pp) = ph;
            *reinterpret_cast<u32x4*>(pp + 16) = pl;
          }
        }
      } else {
        if (t0 < ntl) {
          u32x4 ph, pl;
          make_p(z0, mref, l_add, ph, pl);
          uint8_t* pp = plds + ((t0 * G + my_hg) * 64 + lane) * kPBytes;
          *reinterpret_cast<u32x4*>(pp) = ph;
          *reinterpret_cast<u32x4*>(pp + 16) = pl;
        }
        if (G == 4 && t1 < ntl) {
          u32x4 ph, pl;
          make_p(z1, mref, l_add, ph, pl);
          uint8_t* pp = plds + ((t1 * G + my_hg) * 64 + lane) * kPBytes;
          *reinterpret_cast<u32x4*>(pp) = ph;
          *reinterpret_cast<u32x4*>(pp + 16) = pl;
        }
      }
      return l_add;
    };
    float l_add = write_p(my_m);
    barrier_lds();   // batch maxima and P of every unit in LDS

    // ---- per-group batch max of head n (the same in every wave, so the branch below
    // is uniform over the workgroup) ----
    float fac[G];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mb = m_part[h * 16 + n];   // over the waves of group h: h, h + G, ...
#pragma unroll
      for (int i = 1; i < WPG; ++i) mb = fmaxf(mb, m_part[(h + G * i) * 16 + n]);
      const float m_new = mb > m_run[h] + kLazy ? mb : m_run[h];   // lazy, as above
      fac[h] = (m_run[h] == -INFINITY || m_new == m_run[h]) ? 1.f : __builtin_amdgcn_exp2f(m_run[h] - m_new);
      moved = moved || m_new != m_run[h];
      m_run[h] = m_new;
    }
    if (__any(moved)) {
      float my_fac = fac[0];
      my_m = m_run[0];
#pragma unroll
      for (int h = 1; h < G; ++h) {
        my_fac = my_hg == h ? fac[h] : my_fac;
        my_m = my_hg == h ? m_run[h] : my_m;
      }
      l_part *= my_fac;
      l_add = write_p(my_m);
      // rescale: acc[h][t][i] belongs to head 4g+i of group h, factor in lane 4g+i
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float fo[4];
        bool any = false;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          fo[ii] = __shfl(fac[h], 4 * g + ii, kWave);
          any = any || fo[ii] != 1.f;
        }
        if (__any(any)) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[h][tt][ii] *= fo[ii];
        }
      }
      barrier_lds();   // P written again by every wave
    }
    l_part += l_add;

    // ---- PV: convert each tile's rows once, MFMAs for all four head groups ----
#pragma unroll 1
    for (int tile = 0; tile < ntl; ++tile) {
      uint32_t d01[8], d23[8];
      if (is_win) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2 v = lds_ld<u32x2>(buf + (tile * 32 + slot_row(g, j)) * kWinB + 128 * wid + 8 * n);
          d01[j] = v.x;
          d23[j] = v.y;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint8_t* rp = buf + (tile * 32 + slot_row(g, j)) * kRowB;
          const uint32_t c2 = lds_ld<uint16_t>(rp + 32 * wid + 2 * n);
          const float sc = e8m0_scale(rp[256 + 2 * wid + (n >> 3)]);
          d01[j] = fp4x2_to_bf16x2<0>(c2, sc);
          d23[j] = fp4x2_to_bf16x2<1>(c2, sc);
        }
      }
      bf16x8 bf[4];
      bf[0] = __builtin_bit_cast(bf16x8, u32x4{pack_lo(d01[0], d01[1]), pack_lo(d01[2], d01[3]),
                                               pack_lo(d01[4], d01[5]), pack_lo(d01[6], d01[7])});
      bf[1] = __builtin_bit_cast(bf16x8, u32x4{pack_hi(d01[0], d01[1]), pack_hi(d01[2], d01[3]),
                                               pack_hi(d01[4], d01[5]), pack_hi(d01[6], d01[7])});
      bf[2] = __builtin_bit_cast(bf16x8, u32x4{pack_lo(d23[0], d23[1]), pack_lo(d23[2], d23[3]),
                                               pack_lo(d23[4], d23[5]), pack_lo(d23[6], d23[7])});
      bf[3] = __builtin_bit_cast(bf16x8, u32x4{pack_hi(d23[0], d23[1]), pack_hi(d23[2], d23[3]),
                                               pack_hi(d23[4], d23[5]), pack_hi(d23[6], d23[7])});
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint8_t* pp = plds + ((tile * G + h) * 64 + lane) * kPBytes;
        const bf16x8 ph = __builtin_bit_cast(bf16x8, lds_ld<u32x4>(pp));
        const bf16x8 pl = __builtin_bit_cast(bf16x8, lds_ld<u32x4>(pp + 16));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          acc[h][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bf[tt], acc[h][tt], 0, 0, 0);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          acc[h][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bf[tt], acc[h][tt], 0, 0, 0);
      }
    }
    wait_all_vm();   // this wave's copies of batch k+1 have landed
  }

  // ---- softmax denominators (group h: waves h, h + G, ...), output ----
  float l_head = l_part;
  l_head += __shfl_xor(l_head, 16, kWave);
  l_head += __shfl_xor(l_head, 32, kWave);
  if (g == 0) l_w[wid * 16 + n] = l_head;
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      float lh = l_w[h * 16 + 4 * g + ii];
#pragma unroll
      for (int i = 1; i < WPG; ++i) lh += l_w[(h + G * i) * 16 + 4 * g + ii];
      const float inv = lh > 0.f ? __builtin_amdgcn_rcpf(lh) : 0.f;
      *reinterpret_cast<u32x2*>(a.out + (qi * a.H + 16 * G * hq + 16 * h + 4 * g + ii) * CSA2_D_LATENT + 64 * wid +
                                4 * n) = u32x2{pack_bf16x2(acc[h][0][ii] * inv, acc[h][1][ii] * inv),
                                               pack_bf16x2(acc[h][2][ii] * inv, acc[h][3][ii] * inv)};
    }
  }
  if (a.lse && wid < G && g == 0) {
    float s = l_w[wid * 16 + n], m = m_run[0];
#pragma unroll
    for (int i = 1; i < WPG; ++i) s += l_w[(wid + G * i) * 16 + n];
#pragma unroll
    for (int h = 1; h < G; ++h) m = wid == h ? m_run[h] : m;
    a.lse[qi * a.H + 16 * G * hq + 16 * wid + n] = s > 0.f ? (m + log2f(s)) * kLn2 : -INFINITY;
  }
}

// Waves per workgroup of the 16-head kernel.
constexpr int kNw16 = 4;

bool lds_limit_set() {
  static const bool ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_decode_kernel<kNw16>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, Geo16<kNw16>::LDS) == hipSuccess &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_decode_wide_kernel<4>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, GeoW<4>::LDS) == hipSuccess &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_decode_wide_kernel<2>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, GeoW<2>::LDS) == hipSuccess;
  return ok;
}

}  // namespace

bool attention_batch_ready() { return lds_limit_set(); }

int launch_attention_batch(const csa2_cache_t& c, int B, int C, int H, const int32_t* len, bool prefill,
                           const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* win, int W,
                           float sm_scale, uint16_t* out, float* lse, hipStream_t s) {
  if (!lds_limit_set()) return CSA2_EHIP;
  DecArgs a;
  a.lat_codes = c.lat_codes;
  a.lat_scales = c.lat_scales;
  a.block_table = c.block_table;
  a.n_pages = c.n_pages;
  a.max_pages = c.max_pages;
  a.len = len;
  a.q = q;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.win = win;
  a.W = W;
  a.scale_log2 = sm_scale * kLog2e;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.C = C;
  a.H = H;
  a.HG = H / 16;
  a.prefill = prefill ? 1 : 0;
  a.vshift = vis_shift(c);
  const int64_t nq = (int64_t)B * C;
  const int64_t per = (nq + 7) / 8;
  a.q_per_xcd = (int)per;
  // More heads per workgroup read and convert each row once for more heads, but
  // leave fewer workgroups: 64 heads once the queries alone give every CU a couple of
  // workgroups, else 32.
  if (H % 64 == 0 && nq >= kH64MinQueries) {
    const int64_t grid = 8 * per * (H / 64);
    if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
    constexpr int lds4 = GeoW<4>::LDS;
    hipLaunchKernelGGL(sparse_decode_wide_kernel<4>, dim3((unsigned)grid), dim3(kThreads), lds4, s, a);
    return hip_status();
  }
  if (H % 32 == 0) {
    const int64_t grid = 8 * per * (H / 32);
    if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
    constexpr int lds2 = GeoW<2>::LDS;
    hipLaunchKernelGGL(sparse_decode_wide_kernel<2>, dim3((unsigned)grid), dim3(kThreads), lds2, s, a);
    return hip_status();
  }
  const int64_t grid = 8 * per * a.HG;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  constexpr int lds16 = Geo16<kNw16>::LDS;
  hipLaunchKernelGGL(sparse_decode_kernel<kNw16>, dim3((unsigned)grid), dim3(kNw16 * 64), lds16, s, a);
  return hip_status();
}

}  // namespace csa2
