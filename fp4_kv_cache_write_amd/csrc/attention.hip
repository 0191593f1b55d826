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
// Decomposition: one workgroup per (query, group of 16 heads); blockIdx is mapped
// so that the head groups of one query, and neighbouring queries of one sequence,
// run on the same XCD and share its L2 for the gathered rows.  Four waves, one per SIMD, 512 registers each.  All row data
// reaches LDS through global_load_lds_dwordx4 (no registers, everything in flight at
// once), in two phases that reuse one 136 KB staging area:
//   A. the window rows (bf16, 1 KB each, pitch 1040 B) -- they need no index
//      lookups, so their copies start at once while the selected entries' row ids
//      are resolved through the page table;
//   B. the selected FP4 rows (256 code bytes + 16 scale bytes, pitch 272 B), up to
//      512 per pass.
// Within a phase each wave first computes the scores of all its 32-row tiles, takes
// one maximum, then accumulates P.V -- the accumulators are rescaled at most once
// per phase, so they never leave the MFMA accumulator registers inside the loops.
// The waves' softmax states and accumulators are merged through LDS at the end.
//
// Per 32-row tile:
//   QK  D[row][head] via 16x16x32 bf16 MFMA; A = rows (lane: row l%16, dims
//       128g+8s..+7 at k-step s, g = l/16), B = q (lane: head l%16, same dims).
//       FP4 rows become bf16 operands through the hardware convert with the e8m0
//       scale folded in (exact).
//   P   the lane then holds rows {4g..4g+3, 16+4g..16+4g+3} of head l%16 --
//       exactly the K-slots of the P operand of the PV MFMA, so P needs no
//       cross-lane movement.  P enters as a bf16 head plus a bf16 residual (two
//       MFMAs): plain bf16 weights (8 bits) would use most of the 2e-3 error budget
//       on flat softmaxes.
//   PV  O[head][dim] += P . R via 16x16x32 bf16 MFMA, n-tile t holding dims 32n+t
//       for lane column n, so each lane reads one 16-byte run per row and
//       transposes register pairs (v_perm) into the B operand.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = 272;          // FP4 row in LDS: 256 code bytes then 16 scale bytes
constexpr int kWinB = 1040;         // window row in LDS: 1024 bytes + 16 pad
constexpr int kBatchRows = 512;     // FP4 rows staged per pass
constexpr int kWinBatch = 128;      // window rows staged per pass
constexpr int kMaxT = 4;            // 32-row tiles per wave per pass
constexpr int kQStride = 520;       // bf16 per head row of q in LDS (512 + pad)
constexpr int kOStride = 576;       // floats per head row of a wave's merge slot (36 per 32 dims)
constexpr int kOffRows = 0;
constexpr int kStageBytes = kBatchRows * kRowB;           // 139264 >= kWinBatch * kWinB
constexpr int kOffQ = kStageBytes;                        // spare: part of the merge slots
constexpr int kOffRowId = kOffQ + 16 * kQStride * 2;      // 155904
constexpr int kOffSm = kOffRowId + kBatchRows * 4;        // 157952
constexpr int kLdsBytes = kOffSm + (2 * kWaves * 16 + 32) * 4;
static_assert(kWinBatch * kWinB <= kStageBytes, "window batch fits the staging area");
static_assert(kBatchRows / 32 <= kWaves * kMaxT && kWinBatch / 32 <= kWaves * kMaxT, "tiles per wave");
static_assert(kWaves * 16 * kOStride * 4 <= kOffRowId, "merge slots alias the staging and q areas");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

constexpr float kLog2e = 1.4426950408889634f;
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
  int B, C, H, HG, prefill, q_per_xcd;
};

// low halves of a and b -> (a.lo, b.lo); high halves -> (a.hi, b.hi)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

// P operand (bf16 head + bf16 residual) of this lane's 8 scores (log2 units, -inf =
// absent) against the running max m; adds the weights to l_part.
__device__ __forceinline__ void make_p(const float (&z)[8], float m, float& l_part, bf16x8& pa_hi, bf16x8& pa_lo) {
  const float mb = (m == -INFINITY) ? 0.f : m;
  uint32_t phi[4], plo[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float p0 = exp2f(z[j] - mb), p1 = exp2f(z[j + 1] - mb);
    l_part += p0 + p1;
    const uint32_t h0 = f32_to_bf16_rne(p0), h1 = f32_to_bf16_rne(p1);
    const uint32_t r0 = f32_to_bf16_rne(p0 - bf16_to_f32(h0));
    const uint32_t r1 = f32_to_bf16_rne(p1 - bf16_to_f32(h1));
    phi[j >> 1] = h0 | (h1 << 16);
    plo[j >> 1] = r0 | (r1 << 16);
  }
  pa_hi = __builtin_bit_cast(bf16x8, u32x4{phi[0], phi[1], phi[2], phi[3]});
  pa_lo = __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], plo[2], plo[3]});
}

// B operands of 8 n-tiles t0..t0+7 from 8 rows' bf16 pairs: d[k][j] holds dims
// (t0+2k, t0+2k+1) of row-slot j.  Eight independent accumulator chains, P head
// first, then P residual.
__device__ __forceinline__ void pv_quad(f32x4 (&acc)[32], int t0, bf16x8 pa_hi, bf16x8 pa_lo,
                                        const uint32_t (&d)[4][8]) {
  bf16x8 bf[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    bf[2 * k] = __builtin_bit_cast(bf16x8, u32x4{pack_lo(d[k][0], d[k][1]), pack_lo(d[k][2], d[k][3]),
                                                 pack_lo(d[k][4], d[k][5]), pack_lo(d[k][6], d[k][7])});
    bf[2 * k + 1] = __builtin_bit_cast(bf16x8, u32x4{pack_hi(d[k][0], d[k][1]), pack_hi(d[k][2], d[k][3]),
                                                     pack_hi(d[k][4], d[k][5]), pack_hi(d[k][6], d[k][7])});
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[t0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, bf[k], acc[t0 + k], 0, 0, 0);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[t0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, bf[k], acc[t0 + k], 0, 0, 0);
}

// Row slot of K-slot j for lane group g: rows 4g..4g+3, then 16+4g..16+4g+3.
__device__ __forceinline__ int slot_row(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// Scores of an FP4 tile staged in LDS (rows base..base+31 of the batch).
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
      const int e = k & 1;   // two partial sums per row-tile keep four MFMA chains in flight
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

// P.V of an FP4 tile staged in LDS: lane (n, g) reads the 16-byte MX block n of its 8 rows.
__device__ __forceinline__ void fp4_pv(const uint8_t* rows, int base, bf16x8 pa_hi, bf16x8 pa_lo, f32x4 (&acc)[32]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  u32x4 cd[8];
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint8_t* rp = rows + (base + slot_row(g, j)) * kRowB;
    cd[j] = lds_ld<u32x4>(rp + 16 * n);
    sc[j] = e8m0_scale(rp[256 + n]);
  }
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    uint32_t d[4][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      d[0][j] = fp4x2_to_bf16x2<0>(cd[j][qd], sc[j]);
      d[1][j] = fp4x2_to_bf16x2<1>(cd[j][qd], sc[j]);
      d[2][j] = fp4x2_to_bf16x2<2>(cd[j][qd], sc[j]);
      d[3][j] = fp4x2_to_bf16x2<3>(cd[j][qd], sc[j]);
    }
    pv_quad(acc, 8 * qd, pa_hi, pa_lo, d);
  }
}

// Window slot w (position t-W+1+w) holds a row, i.e. w < W and the position is >= 0.
__device__ __forceinline__ bool win_valid(int W, int t, int w) { return w < W && t - (W - 1) + w >= 0; }

// Scores of a window tile staged in LDS (rows base..base+31 of the window batch w0..).
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
    for (int s = 0; s < 8; ++s) {          // all LDS reads of the half first
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

// P.V of a window tile staged in LDS: lane (n, g) reads dims 32n..32n+31 of its 8 rows.
__device__ __forceinline__ void win_pv(const uint8_t* wrows, int base, bf16x8 pa_hi, bf16x8 pa_lo, f32x4 (&acc)[32]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {   // dims 32n + 8ch .. +7
    uint32_t d[4][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 v = lds_ld<u32x4>(wrows + (base + slot_row(g, j)) * kWinB + 64 * n + 16 * ch);
      d[0][j] = v.x;
      d[1][j] = v.y;
      d[2][j] = v.z;
      d[3][j] = v.w;
    }
    pv_quad(acc, 8 * ch, pa_hi, pa_lo, d);
  }
}

// Raise the running max of head l%16 to cover this phase's scores; rescales the
// accumulators (output head 4g+i's factor comes from lane 4g+i) only when needed.
__device__ __forceinline__ void phase_max(const float (&z)[kMaxT][8], float& m_run, float& l_part,
                                          f32x4 (&acc)[32]) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxT; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) tmax = fmaxf(tmax, z[i][j]);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  const bool had = m_run > -INFINITY;   // accumulators hold weights only after a finite max
  float fac = 1.f;
  if (tmax > m_run) {
    fac = had ? exp2f(m_run - tmax) : 0.f;
    l_part *= fac;
    m_run = tmax;
  }
  float fo[4];
  bool any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fo[i] = __shfl(fac, 4 * g + i, kWave);
    const float mh = __shfl(had ? 1.f : 0.f, 4 * g + i, kWave);
    any = any || (fo[i] != 1.f && mh != 0.f);
  }
  if (__builtin_amdgcn_read_exec() && __any(any)) {
#pragma unroll
    for (int tt = 0; tt < 32; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[tt][i] *= fo[i];
    }
  }
}

__global__ __launch_bounds__(kThreads) void sparse_decode_kernel(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* stage = lds + kOffRows;
  int32_t* rowid = reinterpret_cast<int32_t*>(lds + kOffRowId);
  float* m_w = reinterpret_cast<float*>(lds + kOffSm);
  float* l_w = m_w + kWaves * 16;
  float* m_g = l_w + kWaves * 16;
  float* l_g = m_g + 16;

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

  int64_t L = a.len[b];
  if (L < 0) L = 0;
  if (a.prefill) L += ci + 1;   // chunk query ci sits at position prior + ci
  const int n_vis = (int)(L >> 1);
  const int t = (int)L - 1;
  const uint16_t* win_b = a.win + (int64_t)b * (a.prefill ? a.W - 1 + a.C : a.W) * CSA2_D_LATENT;

  // window batch: LDS chunk c (16 bytes) = piece c%65 of row c/65 (piece 64 = pad)
  auto stage_window = [&](int w0, int nw) {
    const int chunks = nw * 65;
    for (int ins = wid; ins * 64 < chunks; ins += kWaves) {
      const int c = ins * 64 + lane;
      const int r = c / 65, piece = c - r * 65;
      if (c < chunks && piece < 64 && win_valid(a.W, t, w0 + r)) {
        const int pos = t - (a.W - 1) + w0 + r;
        const int row = a.prefill ? ci + w0 + r : pos % a.W;
        const uint16_t* src = win_b + (int64_t)row * CSA2_D_LATENT + 8 * piece;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), stage + ins * 1024, 16, 0, 0);
      }
    }
  };
  // FP4 batch: LDS chunk c = piece c%17 of row c/17 (16 code pieces, then the scales).
  // Row ids of 8 copy instructions are read from LDS before any copy is issued.
  auto stage_fp4 = [&](int nrows) {
    const int chunks = nrows * 17;
    const int n_ins = (chunks + 63) >> 6;
    for (int i0 = wid; i0 < n_ins; i0 += 8 * kWaves) {
      int rid[8], piece[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = (i0 + u * kWaves) * 64 + lane;
        const int r = c / 17;
        piece[u] = c - r * 17;
        rid[u] = c < chunks ? rowid[r] : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ins = i0 + u * kWaves;
        if (ins < n_ins && rid[u] >= 0) {
          const uint8_t* src = piece[u] < 16
                                   ? a.lat_codes + (int64_t)rid[u] * CSA2_LAT_CODE_BYTES + 16 * piece[u]
                                   : a.lat_scales + (int64_t)rid[u] * CSA2_LAT_SCALE_BYTES;
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), stage + ins * 1024, 16, 0, 0);
        }
      }
    }
  };

  // ---- start: window batch 0 copies, q fragments, FP4 row ids of batch 0 ----
  const int n_wb = (a.W + kWinBatch - 1) / kWinBatch;
  stage_window(0, min(a.W, kWinBatch));
  // q operand of head hg*16+n: dims 128g + 8s .. +7 for k-step s
  u32x4 qf[16];
  {
    const uint16_t* qp = a.q + (qi * a.H + hg * 16 + n) * CSA2_D_LATENT + 128 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qp + 8 * s);
  }
  const int n_batches = a.topk > 0 ? (a.topk + kBatchRows - 1) / kBatchRows : 0;
  // row ids of batch r0: entry ids first (independent loads), then their pages
  auto resolve_rows = [&](int r0, int nrows) {
    constexpr int RPT = kBatchRows / kThreads;
    int e[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + u * kThreads;
      e[u] = i < nrows ? a.topk_idx[qi * a.topk + r0 + i] : -1;
    }
    int pg[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const bool ok = e[u] >= 0 && e[u] < n_vis && (e[u] >> 6) < a.max_pages;
      pg[u] = ok ? a.block_table[(int64_t)b * a.max_pages + (e[u] >> 6)] : -1;
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int i = tid + u * kThreads;
      if (i < nrows)
        rowid[i] = (pg[u] >= 0 && pg[u] < a.n_pages) ? pg[u] * CSA2_PAGE + (e[u] & (CSA2_PAGE - 1)) : -1;
    }
  };
  resolve_rows(0, min(a.topk, kBatchRows));

  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  float z[kMaxT][8];

  // ---- phase A: window rows ----
  for (int wb = 0; wb < n_wb; ++wb) {
    const int w0 = wb * kWinBatch;
    const int nw = min(a.W - w0, kWinBatch);
    if (wb > 0) {
      __syncthreads();
      stage_window(w0, nw);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int padded = ((nw + 31) >> 5) << 5;
    for (int c = tid; c < padded * 65; c += kThreads) {
      const int r = c / 65;
      if (!win_valid(a.W, t, w0 + r) || r >= nw) *reinterpret_cast<u32x4*>(stage + c * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const int ntl = padded >> 5;
#pragma unroll
    for (int i = 0; i < kMaxT; ++i) {
      const int tile = wid + kWaves * i;
      if (tile < ntl) {
        win_qk(stage, a.W, t, w0, tile * 32, qf, a.scale_log2, z[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[i][j] = -INFINITY;
      }
    }
    phase_max(z, m_run, l_part, acc);
#pragma unroll
    for (int i = 0; i < kMaxT; ++i) {
      const int tile = wid + kWaves * i;
      if (tile < ntl) {
        bf16x8 ph, pl;
        make_p(z[i], m_run, l_part, ph, pl);
        win_pv(stage, tile * 32, ph, pl, acc);
      }
    }
  }

  // ---- phase B: selected FP4 rows ----
  for (int bt = 0; bt < n_batches; ++bt) {
    const int r0 = bt * kBatchRows;
    const int nrows = min(a.topk - r0, kBatchRows);
    __syncthreads();                               // staging area and row ids free
    if (bt > 0) {
      resolve_rows(r0, nrows);
      __syncthreads();
    }
    stage_fp4(nrows);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int padded = ((nrows + 31) >> 5) << 5;
    for (int c = tid; c < padded * 17; c += kThreads) {
      const int r = c / 17;
      if (r >= nrows || rowid[r] < 0) *reinterpret_cast<u32x4*>(stage + c * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const int ntl = padded >> 5;
#pragma unroll
    for (int i = 0; i < kMaxT; ++i) {
      const int tile = wid + kWaves * i;
      if (tile < ntl) {
        fp4_qk(stage, rowid, nrows, tile * 32, qf, a.scale_log2, z[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) z[i][j] = -INFINITY;
      }
    }
    phase_max(z, m_run, l_part, acc);
#pragma unroll
    for (int i = 0; i < kMaxT; ++i) {
      const int tile = wid + kWaves * i;
      if (tile < ntl) {
        bf16x8 ph, pl;
        make_p(z[i], m_run, l_part, ph, pl);
        fp4_pv(stage, tile * 32, ph, pl, acc);
      }
    }
  }
  __syncthreads();

  // ---------------- merge the waves ----------------
  float l_head = l_part;
  l_head += __shfl_xor(l_head, 16, kWave);
  l_head += __shfl_xor(l_head, 32, kWave);
  if (g == 0) {
    m_w[wid * 16 + n] = m_run;
    l_w[wid * 16 + n] = l_head;
  }
  __syncthreads();
  if (tid < 16) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, m_w[w * 16 + tid]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (m_w[w * 16 + tid] > -INFINITY) l += l_w[w * 16 + tid] * exp2f(m_w[w * 16 + tid] - m);
    m_g[tid] = m;
    l_g[tid] = l;
  }
  __syncthreads();
  // Each wave writes its rescaled accumulators to a slot of its own (plain stores;
  // LDS float atomics serialise badly here).  Lane (n, g) holds O[head 4g+i][dim
  // 32n+t] in acc[t][i]; head 4g+i's running max lives in lane 4g+i.  A slot row
  // keeps 36 floats per 32 dims so the 16 lanes of a store hit distinct banks.
  float* slot = reinterpret_cast<float*>(lds) + wid * 16 * kOStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mh = __shfl(m_run, 4 * g + i, kWave);
    const float f = (mh == -INFINITY) ? 0.f : exp2f(mh - m_g[4 * g + i]);
    float* dst = slot + (4 * g + i) * kOStride + 36 * n;
#pragma unroll
    for (int t4 = 0; t4 < 8; ++t4)
      *reinterpret_cast<f32x4*>(dst + 4 * t4) = f32x4{acc[4 * t4][i] * f, acc[4 * t4 + 1][i] * f,
                                                      acc[4 * t4 + 2][i] * f, acc[4 * t4 + 3][i] * f};
  }
  __syncthreads();
  const float* base = reinterpret_cast<const float*>(lds);
  for (int i = tid; i < 16 * CSA2_D_LATENT / 4; i += kThreads) {
    const int h = (4 * i) / CSA2_D_LATENT, d = (4 * i) % CSA2_D_LATENT;
    const int off = h * kOStride + 36 * (d >> 5) + (d & 31);
    f32x4 s4 = *reinterpret_cast<const f32x4*>(base + off);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s4 += *reinterpret_cast<const f32x4*>(base + w * 16 * kOStride + off);
    const float l = l_g[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const uint32_t v0 = f32_to_bf16_rne(s4[0] * inv), v1 = f32_to_bf16_rne(s4[1] * inv);
    const uint32_t v2 = f32_to_bf16_rne(s4[2] * inv), v3 = f32_to_bf16_rne(s4[3] * inv);
    *reinterpret_cast<u32x2*>(a.out + (qi * a.H + hg * 16 + h) * CSA2_D_LATENT + d) =
        u32x2{v0 | (v1 << 16), v2 | (v3 << 16)};
  }
  if (a.lse && tid < 16) {
    const float l = l_g[tid];
    a.lse[qi * a.H + hg * 16 + tid] = l > 0.f ? (m_g[tid] + log2f(l)) * kLn2 : -INFINITY;
  }
}

bool lds_limit_set() {
  static const bool ok = hipFuncSetAttribute(reinterpret_cast<const void*>(sparse_decode_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes) == hipSuccess;
  return ok;
}

}  // namespace

size_t sparse_decode_ws(int B, int H, int topk) {
  (void)B;
  (void)H;
  (void)topk;
  return 0;
}

int launch_gather_attention(const csa2_cache_t& c, int B, int C, int H, const int32_t* len, bool prefill,
                            const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* win,
                            int W, float sm_scale, uint16_t* out, float* lse, hipStream_t s) {
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
  const int64_t per = ((int64_t)B * C + 7) / 8;
  const int64_t grid = 8 * per * a.HG;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  a.q_per_xcd = (int)per;
  hipLaunchKernelGGL(sparse_decode_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
  return hip_status();
}

int launch_sparse_decode(const csa2_cache_t& c, int B, int H, const int32_t* ctx_len,
                         const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* swa,
                         int W, float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t s) {
  (void)ws;
  return launch_gather_attention(c, B, 1, H, ctx_len, false, q, topk_idx, topk, swa, W, sm_scale, out, lse, s);
}

}  // namespace csa2
