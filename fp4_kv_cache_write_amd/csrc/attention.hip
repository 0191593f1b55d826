// Sparse gather-attention: the top-K FP4 latent rows plus the bf16 sliding window,
// one softmax, K = V = the 512-d latent.  Serves one decode query per sequence and,
// in prefill mode, C chunk queries per sequence whose window rows come from the
// caller's array of the chunk's own tokens.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §1.2 (window 128,
// every head shares one 512-d latent) and §2.3.1 (each query attends to the selected
// entries and the layer's window KV together); [P3] "DeepSeek V4.1 Flash
// architecture..." (scores -> weights summing to 1 -> weighted sum of values).
//
// Decomposition.  One workgroup of 8 waves (two per SIMD) per (query, group of 16
// heads, half or quarter of the output dims).  The window is cut into 16-row units
// and the FP4 rows into 32-row tiles, each dealt round robin to the waves; a wave
// takes whole units and tiles: it scores all 512 dims of its rows for the 16 heads,
// keeps its own online softmax state and accumulates its own O[16 heads][its dims].
// Nothing is shared between waves until the end, so the row loop has no workgroup
// barrier; the eight states are merged once through LDS.  The output dims of a
// (query, head group) are split over 2 workgroups (4 when pairs are few): each part
// scores all rows and writes its own dims, so no partial state goes through HBM and
// a launch of 128 pairs fills 256 CUs.
//
// Costs measured on the MI355X set the shape: a 16x16x32 bf16 MFMA takes ~7.4 ns
// of a SIMD, VALU work adds to it rather than overlapping, and one wave per SIMD
// reaches only half the VALU rate of two.  Hence two waves per SIMD (a wave fits in
// 256 registers with half the dims), and VALU work is kept to the FP4 converts, the
// row pairing of the value operand and a short softmax.
//
// Data path.  Rows are copied from HBM straight into a private LDS region of the
// wave (global_load_lds, 16 bytes per lane); the wave waits for them with an explicit
// vmcnt, so its two FP4 tiles are in flight together.  From LDS:
//   QK  D[row][head] with 16x16x32 bf16 MFMAs.  A = rows (lane: row l%16; at k-step
//       s = 4c + u lane group g holds dims 128c + 32g + 8u .. +7; FP4 codes become
//       bf16 through the hardware convert with the e8m0 scale folded in, exact),
//       B = q (lane: head l%16, the same dims; q stays in registers).
//   P   each lane ends with the scores of head l%16 for rows 4g..4g+3 (and
//       16+4g..16+4g+3 in an FP4 tile): exactly the K-slots of the value MFMA's A
//       operand, so P never leaves the lane.  P enters that MFMA as a bf16 head plus
//       a bf16 residual, since plain bf16 weights use most of the 2e-3 error budget
//       on flat softmaxes.
//   PV  n-tile t of lane column n is dim 32n + t: per row a lane reads the 16 bytes
//       of FP4 codes (or 16 bytes of bf16 per 8 dims) of its 32 dims; the convert
//       gives pairs of dims of one row and v_perm pairs rows into the B operand.  A
//       window unit has 16 rows, so its value MFMAs are the 16x16x16 ones.
//   The running maximum is lazy: it moves only when a tile's maximum passes it by
//   more than 2^8 (weights up to 256 are exact in the bf16 split and fp32 sums), so
//   the accumulator is rescaled almost never.
// LDS layouts are swizzled (XOR of the 16-byte chunk index with the row) so that
// both the QK reads (16 rows, same chunk) and the PV reads (one row, 16 chunks) hit
// distinct banks.
//
// Order of loads.  The window's first eight units all go to waves 0-3: wave w loads
// unit w at once, computes it, then its FP4 tiles, then unit w+4; waves 4-7 take
// only FP4 tiles.  (Waves 0-3 issue first on their SIMDs and so run ahead of waves
// 4-7; measured on the MI355X, dealing them the extra work ends the two waves of a
// SIMD closer together, about 1 us sooner per call at 32 x 64 heads.)  Whatever a
// wave loads late is first warmed into L2 with a few dword loads (window rows at the
// start, FP4 rows right after the page lookups), and the late window unit is loaded
// in halves, each into an FP4 slot as soon as that slot's last tile is done.  The row ids of a tile's DMAs are
// gathered from the lanes holding them before any of the DMAs is issued, and the
// operands of the next 128-dim chunk are read from LDS while the current one is
// multiplied.  Every workgroup of a query reads all of the query's rows; measured on
// the MI355X, a stand-alone gather of that pattern takes a few microseconds of the
// call, and the rest is the chain of each wave (ids, page ids, rows, the tiles' work,
// the merge of the wave states).
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kWavesA = 8;
constexpr int kThreadsA = kWavesA * 64;
constexpr int kTile = 32;                              // FP4 rows per tile
constexpr int kUnit = 16;                              // window rows per unit
constexpr int kCodeB = kTile * CSA2_LAT_CODE_BYTES;    // 8192: FP4 codes of a tile
constexpr int kSlotB = kCodeB + kTile * CSA2_LAT_SCALE_BYTES;   // 8704: + scales
constexpr int kSlots = 2;                              // FP4 tiles in flight per wave
constexpr int kRegionB = kSlots * kSlotB;              // 17408 per wave
constexpr int kWinRowB = 2 * CSA2_D_LATENT;            // 1024: a bf16 window row
constexpr int kMaxFtWave = CSA2_MAX_TOPK / kTile / kWavesA;   // 8 FP4 tiles per wave at most
constexpr int kOffQ = kWavesA * kRegionB;              // q of the 16 heads: [16][512] bf16
constexpr int kOffMask = kOffQ + 16 * kWinRowB;        // [8 waves][8] uint32
constexpr int kOffMl = kOffMask + kWavesA * kMaxFtWave * 4;           // m[8][16], l[8][16]
constexpr int kOffPf = kOffMl + 2 * kWavesA * 16 * 4;    // [8 waves][256 B]: landing area of L2 warm-ups
constexpr int kLdsA = kOffPf + kWavesA * 256;
constexpr int kDmaFp4 = 8 + 2;                         // DMA instructions per FP4 tile
constexpr float kLazy = 8.0f;                          // log2 headroom of the lazy maximum
constexpr int64_t kBatchPairs = 512;                   // from here on, the batched kernels
static_assert(kUnit * kWinRowB <= kRegionB, "a window unit fits the region");
static_assert(kSlotB >= (kUnit / 2) * kWinRowB, "half a window unit fits an FP4 slot");
static_assert(16 * 256 * 4 <= kRegionB, "the merge's O[16][256] fits a region");
static_assert(kLdsA <= 160 * 1024, "LDS budget");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(4))) short s16x4;

struct AttnArgs {
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory into LDS: lane l's bytes land at dst + 16 l.
__device__ __forceinline__ void dma16(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 16, 0, 0);
}
// 4 bytes per lane: lane l's bytes land at dst + 4 l.
__device__ __forceinline__ void dma4(const void* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)dst, 4, 0, 0);
}
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x3f70);
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }   // lgkmcnt(0)

// low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

// Row of K-slot j of an FP4 tile for lane group g: rows 4g..4g+3, then 16+4g..16+4g+3.
__device__ __forceinline__ int slot_row(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// LDS position of 16-byte chunk k of row r.  FP4 rows have 16 chunks, window and q
// rows 64; only the low four bits of the chunk index move (each map is its own
// inverse).
__device__ __forceinline__ int swz_fp4(int k, int r) { return k ^ (r & 15); }
__device__ __forceinline__ int swz_win(int k, int r) { return k ^ (((k >> 4) & 3) ^ (r & 15)); }
__device__ __forceinline__ int swz_q(int k, int h) { return k ^ (h & 15); }

// LDS offset of row r of a window unit in a wave's region: rows 0-7 fill FP4 slot 0
// and rows 8-15 start at slot 1, so each half of a unit can be loaded into one slot
// as soon as that slot's last FP4 tile is done.
__device__ __forceinline__ int win_row_off(int r) { return r * kWinRowB + (r >> 3) * (kSlotB - 8 * kWinRowB); }

// 16-byte chunk c of head h's row in the merge's O area: the bits above the 16 bank
// positions and the head's bits 2-3 are folded into the position, so the stores of a
// wave (16 chunks x 4 heads) and the reads (32 consecutive chunks) spread over all banks.
__device__ __forceinline__ int swz_o(int c, int h) { return c ^ ((c >> 4) & 3) ^ (h & 12); }

// Window slot s (position t-W+1+s) holds a row: s < W and the position is >= 0.
__device__ __forceinline__ bool win_valid(int W, int t, int s) { return s < W && t - (W - 1) + s >= 0; }

// The wave's state: O accumulators of its dim quarters (n-tile t = 8*quarter + tt,
// lane (n, g): heads 4g..4g+3 of dim 32n + 8*quarter + tt), the lazy running maximum
// of head n (identical in the 4 lanes of a head) and the lane's share of the sum.
template <int NQ>
struct WaveState {
  f32x4 acc[NQ * 8];
  float m_run, l_part;
};

// J scores of head n (log2 units, -inf = absent) -> lazy max -> P operands (bf16
// head and residual, J/2 dwords each); rescales the state when the max moves.
template <int NQ, int J>
__device__ __forceinline__ void softmax_scores(WaveState<NQ>& S, const float (&z)[J], int g, uint32_t (&ph)[J / 2],
                                               uint32_t (&pl)[J / 2]) {
  float tmax = z[0];
#pragma unroll
  for (int j = 1; j < J; ++j) tmax = fmaxf(tmax, z[j]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  const bool move = tmax > S.m_run + kLazy;   // also true for the first row seen
  if (__any(move)) {
    const float m_new = move ? tmax : S.m_run;
    const float fac = move ? (S.m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(S.m_run - m_new)) : 1.f;
    S.l_part *= fac;
    // acc[t][i] belongs to head 4g+i, whose factor lives in lane 4g+i
    float fo[4];
    bool any = false;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      fo[ii] = __shfl(fac, 4 * g + ii, kWave);
      any = any || fo[ii] != 1.f;
    }
    if (__any(any)) {
#pragma unroll
      for (int t = 0; t < NQ * 8; ++t)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) S.acc[t][ii] *= fo[ii];
    }
    S.m_run = m_new;
  }
  const float mb = S.m_run == -INFINITY ? 0.f : S.m_run;
#pragma unroll
  for (int j = 0; j < J; j += 2) {
    const float p0 = __builtin_amdgcn_exp2f(z[j] - mb), p1 = __builtin_amdgcn_exp2f(z[j + 1] - mb);
    S.l_part += p0 + p1;
    split_pair(p0, p1, ph[j >> 1], pl[j >> 1]);
  }
}

// Value MFMAs of n-tiles 2m and 2m+1 of quarter qi for an FP4 tile (K = 32 rows):
// c[j] = dims (8q + 2m, 8q + 2m + 1) of the row in K-slot j, as a bf16 pair.
template <int NQ>
__device__ __forceinline__ void pv_pair32(WaveState<NQ>& S, int qi, int m, const uint32_t (&c)[8], bf16x8 ph,
                                          bf16x8 pl) {
  const bf16x8 b0 = __builtin_bit_cast(
      bf16x8, u32x4{pack_lo(c[0], c[1]), pack_lo(c[2], c[3]), pack_lo(c[4], c[5]), pack_lo(c[6], c[7])});
  const bf16x8 b1 = __builtin_bit_cast(
      bf16x8, u32x4{pack_hi(c[0], c[1]), pack_hi(c[2], c[3]), pack_hi(c[4], c[5]), pack_hi(c[6], c[7])});
  f32x4& a0 = S.acc[qi * 8 + 2 * m];
  f32x4& a1 = S.acc[qi * 8 + 2 * m + 1];
  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, b0, a0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, b1, a1, 0, 0, 0);
  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, b0, a0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, b1, a1, 0, 0, 0);
}

// The same for a window unit (K = 16 rows, K-slot j = row 4g + j).
template <int NQ>
__device__ __forceinline__ void pv_pair16(WaveState<NQ>& S, int qi, int m, const uint32_t (&c)[4], s16x4 ph,
                                          s16x4 pl) {
  const s16x4 b0 = __builtin_bit_cast(s16x4, u32x2{pack_lo(c[0], c[1]), pack_lo(c[2], c[3])});
  const s16x4 b1 = __builtin_bit_cast(s16x4, u32x2{pack_hi(c[0], c[1]), pack_hi(c[2], c[3])});
  f32x4& a0 = S.acc[qi * 8 + 2 * m];
  f32x4& a1 = S.acc[qi * 8 + 2 * m + 1];
  a0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, b0, a0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, b1, a1, 0, 0, 0);
  a0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, b0, a0, 0, 0, 0);
  a1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, b1, a1, 0, 0, 0);
}

// Two FP4 codes (byte m of `codes`) as a bf16 pair.
__device__ __forceinline__ uint32_t fp4_pair(uint32_t codes, float scale, int m) {
  switch (m) {
    case 0: return fp4x2_to_bf16x2<0>(codes, scale);
    case 1: return fp4x2_to_bf16x2<1>(codes, scale);
    case 2: return fp4x2_to_bf16x2<2>(codes, scale);
    default: return fp4x2_to_bf16x2<3>(codes, scale);
  }
}

struct Slot0 { static constexpr int value = 0; };
struct Slot1 { static constexpr int value = 1; };

template <int NQ>
__global__ __launch_bounds__(kThreadsA) void attn_kernel(AttnArgs a) {
  static_assert(NQ == 1 || NQ == 2, "one or two dim quarters per workgroup");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int ND = 4 / NQ;   // workgroups per (query, head group)

  // XCD-aware mapping: consecutive workgroup ids go to different XCDs; XCD x takes
  // the contiguous query range [x * q_per_xcd, (x+1) * q_per_xcd), all head groups
  // and dim parts, so the workgroups reading the same rows share one L2.
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int per_q = a.HG * ND;
  const int ql = li / per_q;
  const int rem = li - ql * per_q;
  const int hg = rem / ND;
  const int qd0 = (rem - hg * ND) * NQ;   // first dim quarter of this workgroup
  const int64_t qi = (int64_t)xcd * a.q_per_xcd + ql;
  if (ql >= a.q_per_xcd || qi >= (int64_t)a.B * a.C) return;
  const int b = (int)(qi / a.C);
  const int ci = (int)(qi - (int64_t)b * a.C);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  uint8_t* region = lds + w * kRegionB;
  const uint8_t* qlds = lds + kOffQ;
  uint32_t* vmask = reinterpret_cast<uint32_t*>(lds + kOffMask) + w * kMaxFtWave;

  int64_t Lq = a.len[b];
  if (Lq < 0) Lq = 0;
  if (a.prefill) Lq += ci + 1;   // chunk query ci sits at position prior + ci
  const int n_vis = (int)(Lq >> a.vshift);
  const int t = (int)Lq - 1;
  const int W = a.W;
  const uint16_t* win_b = a.win + (int64_t)b * (a.prefill ? W - 1 + a.C : W) * CSA2_D_LATENT;
  const int32_t* tk = a.topk_idx + qi * a.topk;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;

  const int n_wu = (W + kUnit - 1) / kUnit;       // window units; this wave's: w, w + 8, ...
  const int n_ft = (a.topk + kTile - 1) / kTile;  // FP4 tiles; this wave's: w, w + 8, ...
  const int nk = n_ft > w ? (n_ft - w + kWavesA - 1) / kWavesA : 0;

  // ---- prologue: entry ids of this wave's FP4 tiles (lane: tile 2u + lane/32, row
  // lane%32), q, and the first window unit's rows; page lookups follow the ids.
  int ids[kMaxFtWave / 2];
#pragma unroll
  for (int u = 0; u < kMaxFtWave / 2; ++u) {
    ids[u] = -1;
    if (2 * u < nk) {
      const int k = 2 * u + (lane >> 5);
      const int i = kTile * (w + kWavesA * k) + (lane & 31);
      if (k < nk && i < a.topk) ids[u] = tk[i];
    }
  }
  // q of heads 2w, 2w+1 into LDS (row = head, chunk k of 8 dims at swz_q(k, head));
  // every wave reads all 16 heads from there after the barrier below.
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int head = 2 * w + hh;
    dma16(a.q + (qi * a.H + hg * 16 + head) * CSA2_D_LATENT + 8 * swz_q(lane, head),
          lds + kOffQ + head * kWinRowB);
  }
  // B operand of k-step 4c+u: head n, dims 128c + 32g + 8u .. +7, at chunk
  // swz_q(16c + 4g + u, n) = 16c + (xg ^ u) of head n's row, xg = 4g ^ n: four lane
  // bases, the 256c in the instruction's offset.
  const int xg = (4 * g) ^ n;
  const uint8_t* qb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) qb[u] = qlds + n * kWinRowB + 16 * (xg ^ u);
  auto q_op = [&](int c, int u) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, lds_ld<u32x4>(qb[u] + 256 * c));
  };
  // Window unit wu into the region: row r = slot 16wu + r at win_row_off(r).  A slot
  // with no token reads the row of position t (always present) and is masked in the
  // scores.  Rows r0 .. r0+nr-1 of the unit.
  const int row_t = a.prefill ? ci + W - 1 : (t < 0 ? 0 : t % W);
  auto ring_row = [&](int s) __attribute__((always_inline)) {   // array row of slot s if it holds a token
    if (a.prefill) return ci + s;
    const int ring = (t - (W - 1) + s) % W;
    return ring < 0 ? ring + W : ring;
  };
  auto win_row = [&](int s) __attribute__((always_inline)) { return win_valid(W, t, s) ? ring_row(s) : row_t; };
  auto dma_window_rows = [&](int wu, int r0, int nr) __attribute__((always_inline)) {
    const int s0 = kUnit * wu + r0;
    int row = ring_row(s0);   // advanced by one per slot
#pragma unroll 4
    for (int r = 0; r < nr; ++r) {
      const int s = s0 + r;
      const int rw = win_valid(W, t, s) ? row : row_t;
      dma16(win_b + (int64_t)rw * CSA2_D_LATENT + 8 * swz_win(lane, r0 + r), region + win_row_off(r0 + r));
      row = a.prefill ? row + 1 : (row + 1 == W ? 0 : row + 1);
    }
  };
  auto dma_window = [&](int wu) __attribute__((always_inline)) { dma_window_rows(wu, 0, kUnit); };
  // L2 warm-up of window unit wu (128 lines of 128 bytes; two dword loads per lane whose
  // bytes land in this wave's scratch area, which nothing reads)
  auto warm_window = [&](int wu) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int line = 64 * i + lane;
      dma4(win_b + (int64_t)win_row(kUnit * wu + (line >> 3)) * CSA2_D_LATENT + 64 * (line & 7),
           lds + kOffPf + 256 * w);
    }
  };
  // Waves w and w+4 share a SIMD.  Waves 0-3 take window unit w first and waves 4-7
  // their FP4 tiles, so one of each pair computes while the other waits for its rows;
  // waves 0-3 also take unit w+4 after their tiles.
  const bool win_first = w < 4;
  const bool has_win = win_first && w < n_wu;    // unit w before the FP4 tiles
  const int late_wu = w + 4;                     // and unit w + 4 after them
  const bool late_win = win_first && late_wu < n_wu;
  if (has_win) dma_window(w);
  if (late_win) warm_window(late_wu);
  // ids and q have landed; the window rows and warm-ups issued after them may still be
  // in flight (the barrier does not wait for waves 0-3's window rows)
  if (has_win && late_win)
    wait_vm<kUnit + 2>();
  else if (has_win)
    wait_vm<kUnit>();
  else if (late_win)
    wait_vm<2>();
  else
    wait_vm<0>();
  // q of every head is in LDS.  A bare barrier: the fence of __syncthreads would wait
  // for every load in flight, the window rows included.
  asm volatile("s_barrier" ::: "memory");

  // page lookups of the ids: one load per pair of tiles, issued whatever the lanes
  // hold (an invalid id reads the table's first slot and is dropped), so their number
  // is known to the waits below
  int pg[kMaxFtWave / 2];   // the raw table slot; validity is applied where it is used
  int n_pl = 0;
#pragma unroll
  for (int u = 0; u < kMaxFtWave / 2; ++u) {
    pg[u] = -1;
    if (2 * u < nk) {
      const int e = ids[u];
      const bool ok = e >= 0 && e < n_vis && (e >> 6) < a.max_pages;
      pg[u] = bt[ok ? e >> 6 : 0];
      ++n_pl;
    }
  }
  // waves 0-3: their window unit's rows (issued before the warm-ups and the lookups)
  if (has_win) {
    switch (n_pl + (late_win ? 2 : 0)) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<1>(); break;
      case 2: wait_vm<2>(); break;
      case 3: wait_vm<3>(); break;
      case 4: wait_vm<4>(); break;
      case 5: wait_vm<5>(); break;
      default: wait_vm<6>(); break;
    }
  }

  WaveState<NQ> S;
#pragma unroll
  for (int i = 0; i < NQ * 8; ++i) S.acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  S.m_run = -INFINITY;
  S.l_part = 0.f;

  // ---- a window unit: 16 rows, QK with 16 MFMAs, value MFMAs with K = 16 ----
  auto window_unit = [&](int wu) __attribute__((always_inline)) {
    const int s0 = kUnit * wu;
    float z[4];
    {
      f32x4 sa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      // row n's chunk swz_win(16c + 4g + u, n) = 16c + (xg ^ (u ^ c)): four lane bases
      const uint8_t* rp = region + win_row_off(n);
      const uint8_t* wb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) wb[kk] = rp + 16 * (xg ^ kk);
      // chunk c: row n's dims 128c + 32g + 8u .. +7 and q's k-steps; chunk c+1's reads
      // are issued before chunk c's products (the unit often runs with its SIMD's other
      // wave idle, so nothing else hides the LDS latency)
      struct WinIn {
        u32x4 v[4], q[4];
      };
      auto win_load = [&](int c) __attribute__((always_inline)) {
        WinIn in;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          in.v[u] = lds_ld<u32x4>(wb[u ^ c] + 256 * c);
          in.q[u] = __builtin_bit_cast(u32x4, q_op(c, u));
        }
        return in;
      };
      WinIn cur = win_load(0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        WinIn nxt;
        if (c < 3) nxt = win_load(c + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          sa[u & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.v[u]),
                                                              __builtin_bit_cast(bf16x8, cur.q[u]), sa[u & 1], 0, 0, 0);
        if (c < 3) cur = nxt;
        __builtin_amdgcn_sched_barrier(0);
      }
      const f32x4 sv = sa[0] + sa[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = win_valid(W, t, s0 + 4 * g + j) ? sv[j] * a.scale_log2 : -INFINITY;
    }
    // value operands (rows 4g..4g+3, this lane's dims of each quarter), read before the
    // softmax so their latency overlaps it
    u32x4 v[NQ][4];
#pragma unroll
    for (int qi2 = 0; qi2 < NQ; ++qi2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g + j;
        v[qi2][j] = lds_ld<u32x4>(region + win_row_off(r) + 16 * swz_win(4 * n + qd0 + qi2, r));
      }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t ph[2], pl[2];
    softmax_scores<NQ, 4>(S, z, g, ph, pl);
    const s16x4 phv = __builtin_bit_cast(s16x4, u32x2{ph[0], ph[1]});
    const s16x4 plv = __builtin_bit_cast(s16x4, u32x2{pl[0], pl[1]});
#pragma unroll
    for (int qi2 = 0; qi2 < NQ; ++qi2) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t c[4] = {v[qi2][0][m], v[qi2][1][m], v[qi2][2][m], v[qi2][3][m]};
        pv_pair16<NQ>(S, qi2, m, c, phv, plv);
      }
    }
  };
  if (has_win) window_unit(w);

  // row ids of the FP4 tiles stay in registers (lane: tile 2u + lane/32, row
  // lane%32); vmask[k] bit r = row r of tile k valid
  int rowv[kMaxFtWave / 2];
#pragma unroll
  for (int u = 0; u < kMaxFtWave / 2; ++u) {
    rowv[u] = -1;
    if (2 * u < nk) {
      const int e = ids[u], p = pg[u];
      const bool ok = e >= 0 && e < n_vis && (e >> 6) < a.max_pages && p >= 0 && p < a.n_pages;
      rowv[u] = ok ? p * CSA2_PAGE + (e & (CSA2_PAGE - 1)) : -1;
      const uint64_t bal = __ballot(rowv[u] >= 0);
      if (lane == 0) {
        vmask[2 * u] = (uint32_t)bal;
        if (2 * u + 1 < nk) vmask[2 * u + 1] = (uint32_t)(bal >> 32);
      }
    }
  }
  // The page lookups have all been consumed; saying so here keeps the compiler from
  // waiting for every load in flight (the FP4 tiles' DMAs) at the FP4 loop's entry.
  wait_vm<0>();
  // Waves 0-3 load their FP4 rows only after their window unit: warm those rows' lines
  // into L2 now (codes: two lines per row, scales: one).
  if (win_first) {
#pragma unroll
    for (int u = 0; u < kMaxFtWave / 2; ++u) {
      if (2 * u < nk) {
        const int rr = rowv[u];
        const uint8_t* cp = rr >= 0 ? a.lat_codes + (int64_t)rr * CSA2_LAT_CODE_BYTES : (const uint8_t*)a.q;
        const uint8_t* sp = rr >= 0 ? a.lat_scales + (int64_t)rr * CSA2_LAT_SCALE_BYTES : (const uint8_t*)a.q;
        dma4(cp, lds + kOffPf + 256 * w);
        dma4(cp + 128, lds + kOffPf + 256 * w);
        dma4(sp, lds + kOffPf + 256 * w);
      }
    }
  }
  // the window units this wave has not done yet: beyond the first, for windows longer
  // than 128 (waves 4-7 load their first unit in halves as their FP4 slots free up)
  auto rest_of_window = [&]() __attribute__((always_inline)) {
    for (int wu = w + kWavesA; wu < n_wu; wu += kWavesA) {
      wait_lds();
      dma_window(wu);
      wait_vm<0>();
      window_unit(wu);
    }
  };
  if (win_first) rest_of_window();
  wait_lds();   // the region is free, the validity masks are stored

  // ---- FP4 tiles: two slots, each refilled two tiles ahead ----
  // A row with no entry reads q's first bytes (always present) and is masked: its
  // score is -inf and its value scale is replaced by 0, so its codes stay finite.
  // The row of each of tile k's ten DMAs, fetched from the lanes holding them (all
  // shuffles first, then the DMAs, so their latencies are not paid one by one).
  struct Fp4Rows {
    int r[10];
  };
  auto fp4_rows = [&](int k) __attribute__((always_inline)) {
    const int u = k >> 1, hk = 32 * (k & 1);
    int rw = rowv[0];
#pragma unroll
    for (int uu = 1; uu < kMaxFtWave / 2; ++uu) rw = u == uu ? rowv[uu] : rw;
    Fp4Rows fr;
#pragma unroll
    for (int i = 0; i < 8; ++i) fr.r[i] = __shfl(rw, hk + 4 * i + (lane >> 4), kWave);   // codes: rows 4i + lane/16
#pragma unroll
    for (int i = 0; i < 2; ++i) fr.r[8 + i] = __shfl(rw, hk + 16 * i + (lane >> 2), kWave);   // scales: 16i + lane/4
    return fr;
  };
  auto fp4_dma = [&](const Fp4Rows& fr, uint8_t* slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4), rr = fr.r[i];
      const void* src = rr >= 0 ? (const void*)(a.lat_codes + (int64_t)rr * CSA2_LAT_CODE_BYTES + 16 * swz_fp4(lane & 15, r))
                                : (const void*)a.q;
      dma16(src, slot + 1024 * i);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = fr.r[8 + i];
      const void* src = rr >= 0 ? (const void*)(a.lat_scales + (int64_t)rr * CSA2_LAT_SCALE_BYTES + 4 * (lane & 3))
                                : (const void*)a.q;
      dma4(src, slot + kCodeB + 256 * i);
    }
  };
  auto dma_fp4 = [&](int k, uint8_t* slot) __attribute__((always_inline)) {
    const Fp4Rows fr = fp4_rows(k);
    __builtin_amdgcn_sched_barrier(0);
    fp4_dma(fr, slot);
  };
  if (nk > 1) {   // both tiles' shuffles, then both tiles' DMAs
    const Fp4Rows f0 = fp4_rows(0), f1 = fp4_rows(1);
    __builtin_amdgcn_sched_barrier(0);
    fp4_dma(f0, region);
    fp4_dma(f1, region + kSlotB);
  } else if (nk == 1) {
    dma_fp4(0, region);
  }
  if (nk <= 1 && late_win) dma_window_rows(late_wu, kUnit / 2, kUnit / 2);   // slot 1 holds no tile
  if (nk == 0 && late_win) dma_window_rows(late_wu, 0, kUnit / 2);

  // one FP4 tile from slot SL (a compile-time constant, so LDS offsets are immediates)
  auto fp4_tile = [&](int k, auto slot_c) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const uint8_t* slot = region + SL * kSlotB;
    // validity of rows 4g + j (bit j) and 16 + 4g + j (bit 16 + j)
    const uint32_t vmg = __builtin_amdgcn_readfirstlane(vmask[k]) >> (4 * g);
    float z[8];
    {
      f32x4 sa[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      // operands of chunk c: rows n and 16+n, 16 code bytes each (dims 128c + 32g .. +31),
      // the scale dwords holding that block's byte (byte g of dword c), and q's four
      // k-steps; chunk c+1's are read while chunk c is multiplied
      struct QkIn {
        u32x4 c0, c1, q[4];
        uint32_t s0w, s1w;
      };
      auto qk_load = [&](int c) __attribute__((always_inline)) {
        QkIn in;
        in.c0 = lds_ld<u32x4>(slot + n * CSA2_LAT_CODE_BYTES + 16 * swz_fp4(4 * c + g, n));
        in.c1 = lds_ld<u32x4>(slot + (16 + n) * CSA2_LAT_CODE_BYTES + 16 * swz_fp4(4 * c + g, n));
        in.s0w = lds_ld<uint32_t>(slot + kCodeB + n * CSA2_LAT_SCALE_BYTES + 4 * c);
        in.s1w = lds_ld<uint32_t>(slot + kCodeB + (16 + n) * CSA2_LAT_SCALE_BYTES + 4 * c);
#pragma unroll
        for (int u = 0; u < 4; ++u) in.q[u] = __builtin_bit_cast(u32x4, q_op(c, u));
        return in;
      };
      QkIn cur = qk_load(0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        QkIn nxt;
        if (c < 3) nxt = qk_load(c + 1);
        __builtin_amdgcn_sched_barrier(0);   // keep chunk c+1's reads ahead of chunk c's products
        const float sc0 = e8m0_scale(__builtin_amdgcn_ubfe(cur.s0w, 8 * g, 8));
        const float sc1 = e8m0_scale(__builtin_amdgcn_ubfe(cur.s1w, 8 * g, 8));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 qv = __builtin_bit_cast(bf16x8, cur.q[u]);
          sa[u & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fp4x8_to_bf16x8(cur.c0[u], sc0)),
                                                              qv, sa[u & 1], 0, 0, 0);
          sa[2 + (u & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, fp4x8_to_bf16x8(cur.c1[u], sc1)), qv, sa[2 + (u & 1)], 0, 0, 0);
        }
        if (c < 3) cur = nxt;
        __builtin_amdgcn_sched_barrier(0);
      }
      const f32x4 s0v = sa[0] + sa[1], s1v = sa[2] + sa[3];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        z[j] = ((vmg >> j) & 1u) ? s0v[j] * a.scale_log2 : -INFINITY;
        z[4 + j] = ((vmg >> (16 + j)) & 1u) ? s1v[j] * a.scale_log2 : -INFINITY;
      }
    }
    uint32_t ph[4], pl[4];
    softmax_scores<NQ, 8>(S, z, g, ph, pl);
    const bf16x8 phv = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
    const bf16x8 plv = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});

    // value operand: the lane's code dwords of its dims 32n + 8*qd0 .. + 8*NQ in each
    // of its 8 rows (dword qi of row j = dims 32n + 8(qd0 + qi) .. +7)
    uint32_t v[8][NQ];
    float scf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = slot_row(g, j);
      const uint8_t* cp = slot + r * CSA2_LAT_CODE_BYTES + 16 * swz_fp4(n, r) + 4 * qd0;
      if constexpr (NQ == 1) {
        v[j][0] = lds_ld<uint32_t>(cp);
      } else {
        const u32x2 d = lds_ld<u32x2>(cp);
        v[j][0] = d.x;
        v[j][1] = d.y;
      }
      const uint32_t u8 = slot[kCodeB + r * CSA2_LAT_SCALE_BYTES + n];
      const uint32_t ok = (vmg >> (j < 4 ? j : 12 + j)) & 1u;
      scf[j] = e8m0_scale(u8 & (0u - ok));   // absent row: scale byte 0, finite, weight 0
    }
#pragma unroll
    for (int qi2 = 0; qi2 < NQ; ++qi2) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = fp4_pair(v[j][qi2], scf[j], m);
        pv_pair32<NQ>(S, qi2, m, c, phv, plv);
      }
    }
  };
  // Wait for tile j: the only loads issued after tile j's are the next tile's, or a
  // half window unit loaded into a slot whose tiles are done (waves 4-7).
  auto wait_tile = [&](int j) __attribute__((always_inline)) {
    if (j + 1 < nk)
      wait_vm<kDmaFp4>();
    else if (late_win && (j >= 1 || nk == 1))
      wait_vm<kUnit / 2>();
    else
      wait_vm<0>();
  };
  for (int k = 0; k < nk; k += 2) {
    wait_tile(k);   // tile k landed; k+1 may be in flight
    fp4_tile(k, Slot0{});
    if (k + 2 < nk) {
      wait_lds();   // every read of slot 0 has returned
      dma_fp4(k + 2, region);
    } else if (late_win) {
      wait_lds();
      dma_window_rows(late_wu, 0, kUnit / 2);
    }
    if (k + 1 < nk) {
      wait_tile(k + 1);
      fp4_tile(k + 1, Slot1{});
      if (k + 3 < nk) {
        wait_lds();
        dma_fp4(k + 3, region + kSlotB);
      } else if (late_win) {
        wait_lds();
        dma_window_rows(late_wu, kUnit / 2, kUnit / 2);
      }
    }
  }
  if (late_win) {
    wait_vm<0>();
    window_unit(late_wu);
  }

  if (!win_first) rest_of_window();

  // ---- merge the eight waves: m, l to LDS; O into the wave's own region ----
  float l_head = S.l_part;
  l_head += __shfl_xor(l_head, 16, kWave);
  l_head += __shfl_xor(l_head, 32, kWave);
  float* m_all = reinterpret_cast<float*>(lds + kOffMl);
  float* l_all = m_all + kWavesA * 16;
  if (g == 0) {
    m_all[w * 16 + n] = S.m_run;
    l_all[w * 16 + n] = l_head;
  }
  wait_lds();
  float* ow = reinterpret_cast<float*>(region);   // [16 heads][NQ*128 dims of this part]
  constexpr int kDimsP = NQ * 128;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
#pragma unroll
    for (int qi2 = 0; qi2 < NQ; ++qi2) {
      const int h = 4 * g + ii, c = 2 * (n * NQ + qi2);   // local dims 4c .. 4c+7
      float* row = ow + h * kDimsP;
      *reinterpret_cast<f32x4*>(row + 4 * swz_o(c, h)) = f32x4{S.acc[qi2 * 8 + 0][ii], S.acc[qi2 * 8 + 1][ii],
                                                             S.acc[qi2 * 8 + 2][ii], S.acc[qi2 * 8 + 3][ii]};
      *reinterpret_cast<f32x4*>(row + 4 * swz_o(c + 1, h)) = f32x4{S.acc[qi2 * 8 + 4][ii], S.acc[qi2 * 8 + 5][ii],
                                                                 S.acc[qi2 * 8 + 6][ii], S.acc[qi2 * 8 + 7][ii]};
    }
  __syncthreads();

  // wave w writes heads 2w, 2w+1: lane (m = lane%32, head 2w + lane/32) covers local
  // dims [4*NQ*m, 4*NQ*(m+1)) = output dims 32(m/2) + 8*qd0 + 4*NQ*(m%2) .. + 4*NQ
  constexpr int kPer = 4 * NQ;
  const int head = 2 * w + (lane >> 5), m = lane & 31;
  f32x4 part[kWavesA][kPer / 4];   // every read issued before the first is used
#pragma unroll
  for (int v2 = 0; v2 < kWavesA; ++v2) {
    const float* src = reinterpret_cast<const float*>(lds + v2 * kRegionB) + head * kDimsP;
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i)
      part[v2][i] = *reinterpret_cast<const f32x4*>(src + 4 * swz_o((kPer / 4) * m + i, head));
  }
  float mw[kWavesA], lw[kWavesA], M = -INFINITY;
#pragma unroll
  for (int v2 = 0; v2 < kWavesA; ++v2) {
    mw[v2] = m_all[v2 * 16 + head];
    lw[v2] = l_all[v2 * 16 + head];
    M = fmaxf(M, mw[v2]);
  }
  float o[kPer], L = 0.f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) o[i] = 0.f;
#pragma unroll
  for (int v2 = 0; v2 < kWavesA; ++v2) {
    const float fw = mw[v2] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[v2] - M);
    L += fw * lw[v2];
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * i + e] += fw * part[v2][i][e];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* op = a.out + (qi * a.H + hg * 16 + head) * CSA2_D_LATENT + 32 * (m >> 1) + 8 * qd0 + kPer * (m & 1);
  if constexpr (kPer == 4) {
    *reinterpret_cast<u32x2*>(op) = u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
  } else {
#pragma unroll
    for (int i = 0; i < kPer / 8; ++i) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pk[e] = pack_bf16x2(o[8 * i + 2 * e] * inv, o[8 * i + 2 * e + 1] * inv);
      *reinterpret_cast<u32x4*>(op + 8 * i) = pk;
    }
  }
  if (a.lse && qd0 == 0 && m == 0)
    a.lse[qi * a.H + hg * 16 + head] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

bool lds_limit_set() {
  static const bool ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(attn_kernel<1>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsA) == hipSuccess &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(attn_kernel<2>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          kLdsA) == hipSuccess;
  return ok;
}

}  // namespace

bool attention_kernels_ready() { return lds_limit_set() && attention_batch_ready(); }

size_t sparse_decode_ws(int B, int H, int topk) {
  (void)B;
  (void)H;
  (void)topk;
  return 0;
}

int launch_gather_attention(const csa2_cache_t& c, int B, int C, int H, const int32_t* len, bool prefill,
                            const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* win,
                            int W, float sm_scale, uint16_t* out, float* lse, hipStream_t s, void* ws,
                            size_t ws_bytes) {
  (void)ws;
  (void)ws_bytes;
  if (!lds_limit_set()) return CSA2_EHIP;
  if (topk > CSA2_MAX_TOPK || W < 1 || W > CSA2_MAX_WINDOW) return CSA2_EINVAL;
  // Launches with 512 or more (query, head group) pairs fill every CU for several
  // rounds: there the batched kernels' throughput wins over the short latency
  // chain of the kernel below (measured: 128 x 64-head decode 54 against 67 us,
  // 16384-query prefill attention about 2.5x faster).
  if ((int64_t)B * C * (H / 16) >= kBatchPairs)
    return launch_attention_batch(c, B, C, H, len, prefill, q, topk_idx, topk, win, W, sm_scale, out, lse, s);
  AttnArgs a;
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
  // The output dims of a (query, head group) go to 2 workgroups, or to 4 while the
  // pairs alone would leave most CUs idle.
  const int64_t pairs = nq * a.HG;
  const int nqrt = pairs >= 128 ? 2 : 1;
  const int64_t grid = 8 * per * a.HG * (4 / nqrt);
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  if (nqrt == 2)
    hipLaunchKernelGGL(attn_kernel<2>, dim3((unsigned)grid), dim3(kThreadsA), kLdsA, s, a);
  else
    hipLaunchKernelGGL(attn_kernel<1>, dim3((unsigned)grid), dim3(kThreadsA), kLdsA, s, a);
  return hip_status();
}

int launch_sparse_decode(const csa2_cache_t& c, int B, int H, const int32_t* ctx_len,
                         const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* swa,
                         int W, float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                         hipStream_t s) {
  return launch_gather_attention(c, B, 1, H, ctx_len, false, q, topk_idx, topk, swa, W, sm_scale, out, lse, s,
                                 ws, ws_bytes);
}

}  // namespace csa2
