// Sparse gather-attention for one decode query per sequence: the top-K FP4 latent
// rows plus the bf16 sliding window, one softmax, K = V = the 512-d latent.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §1.2 (window 128,
// every head shares one 512-d latent) and §2.3.1 (each query attends to the selected
// entries and the layer's window KV together); [P3] "DeepSeek V4.1 Flash
// architecture..." (scores -> weights summing to 1 -> weighted sum of values).
//
// Decomposition: one workgroup per (sequence, group of 16 heads); blockIdx is mapped
// so that the head groups of one sequence run on the same XCD and share its L2 for
// the gathered rows.  Per workgroup (4 waves, one per SIMD, 512 registers each):
//   1. the selected entries' row ids go to LDS, and so does q (16 heads x 512);
//   2. every selected FP4 row (256 code bytes + 16 scale bytes) is copied straight
//      from the paged cache into LDS with global_load_lds_dwordx4 -- up to 512 rows,
//      139 KB, all in flight at once and without touching registers;
//   3. while those copies land, the window rows (bf16) are processed from global
//      memory;
//   4. the FP4 rows are processed from LDS, 32-row tiles dealt round-robin to waves;
//   5. the waves' softmax states and accumulators are merged through LDS.
//
// Per 32-row tile a wave runs:
//   QK  D[row][head] via 16x16x32 bf16 MFMA; A = rows (lane: row l%16, dims
//       128g+8s..+7 at k-step s, g = l/16), B = q (lane: head l%16, same dims).
//       FP4 rows become bf16 operands through the hardware convert with the e8m0
//       scale folded in (exact).
//   softmax  the lane then holds rows {4g..4g+3, 16+4g..16+4g+3} of head l%16 --
//       exactly the K-slots of the P operand of the next MFMA, so P needs no
//       cross-lane movement.  The running maximum is only raised when a tile
//       exceeds it by 2^8, which bounds p by 256 and spares rescaling the
//       accumulators on almost every tile; the result is exact either way.
//   PV  O[head][dim] += P . R via 16x16x32 bf16 MFMA, n-tile t holding dims 32n+t
//       for lane column n, so each lane reads one 16-byte MX block per row and
//       transposes register pairs into the B operand.  P enters as a bf16 head plus
//       a bf16 residual (two MFMAs): plain bf16 weights (8 bits) would use most of
//       the 2e-3 error budget on flat softmaxes.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowB = 272;          // LDS row: 256 code bytes then 16 scale bytes
constexpr int kBatchRows = 512;     // FP4 rows staged per pass
constexpr int kQStride = 520;       // bf16 per head row of q in LDS (512 + pad)
constexpr int kOStride = 576;       // floats per head row of a wave's merge slot (36 per 32 dims)
constexpr int kOffRows = 0;
constexpr int kOffQ = kBatchRows * kRowB;                 // 139264
constexpr int kOffRowId = kOffQ + 16 * kQStride * 2;      // 155904
constexpr int kOffSm = kOffRowId + kBatchRows * 4;        // 157952
constexpr int kLdsBytes = kOffSm + (2 * kWaves * 16 + 32) * 4;
static_assert(kWaves * 16 * kOStride * 4 <= kOffRowId, "merge slots alias the row and q areas");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;

struct DecArgs {
  const uint8_t* lat_codes;
  const uint8_t* lat_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* ctx_len;
  const uint16_t* q;
  const int32_t* topk_idx;
  int topk;
  const uint16_t* swa;
  int W;
  float scale_log2;   // sm_scale * log2(e)
  uint16_t* out;
  float* lse;
  int B, H, HG;
};

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t* p) { return *reinterpret_cast<const T*>(p); }

// Cache row (page * 64 + slot) of selection slot i, or -1 when absent.
__device__ __forceinline__ int32_t fp4_row_id(const DecArgs& a, int b, int n_vis, int i) {
  if (i >= a.topk) return -1;
  const int e = a.topk_idx[(int64_t)b * a.topk + i];
  if (e < 0 || e >= n_vis) return -1;
  const int page = page_of(a.block_table, a.max_pages, a.n_pages, b, e);
  if (page < 0) return -1;
  return page * CSA2_PAGE + (e & (CSA2_PAGE - 1));
}

// Window row of window slot w (pos = t-W+1+w) in swa, or -1.
__device__ __forceinline__ int64_t win_row(const DecArgs& a, int b, int t, int w) {
  if (w >= a.W) return -1;
  const int pos = t - (a.W - 1) + w;
  if (pos < 0) return -1;
  return (int64_t)b * a.W + (pos % a.W);
}

struct Softmax {
  float m_run;   // running max (log2 units) of head l%16
  float l_part;  // this lane's share of that head's denominator
};

// Online-softmax update for one tile: z[8] are this lane's scores (log2 units,
// -inf = absent) of head l%16; returns the P operand (hi, lo) and rescales acc.
__device__ __forceinline__ void softmax_tile(float (&z)[8], Softmax& st, f32x4 (&acc)[32], bf16x8& pa_hi,
                                             bf16x8& pa_lo) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  float tmax = z[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, z[j]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
  // The accumulators of output head h sit in lanes with 4g+i == h, so each lane
  // fetches the factors of its 4 output heads from the softmax lanes 4g+i.
  float fac = 1.f;
  if (tmax > st.m_run + kLazy || (st.m_run == -INFINITY && tmax > -INFINITY)) {
    fac = (st.m_run == -INFINITY) ? 0.f : exp2f(st.m_run - tmax);
    st.l_part *= fac;
    st.m_run = tmax;
  }
  float fo[4];
  bool any = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fo[i] = __shfl(fac, 4 * g + i, kWave);
    any = any || (fo[i] != 1.f);
  }
  if (any) {
#pragma unroll
    for (int tt = 0; tt < 32; ++tt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[tt][i] *= fo[i];
    }
  }
  const float mb = (st.m_run == -INFINITY) ? 0.f : st.m_run;
  uint32_t phi[4], plo[4];
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float p0 = exp2f(z[j] - mb), p1 = exp2f(z[j + 1] - mb);
    st.l_part += p0 + p1;
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

// One 32-row tile of FP4 rows staged in LDS (rows base..base+31 of the batch).
__device__ __forceinline__ void fp4_tile(const uint8_t* rows, const int32_t* rowid, int nrows, int base,
                                         const uint16_t* qs, float scale_log2, Softmax& st, f32x4 (&acc)[32]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  // QK: A rows base + 16h + n, B = q head n; k-step s = 4c + k covers dims 128g + 8s.
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
  const uint16_t* qrow = qs + n * kQStride + 128 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float sc0 = e8m0_scale((sb0 >> (8 * c)) & 0xffu);
    const float sc1 = e8m0_scale((sb1 >> (8 * c)) & 0xffu);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * c + k)));
      const int e = k & 1;   // two partial sums per row-tile keep four MFMA chains in flight
      sa[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fp4x8_to_bf16x8(cd0[c][k], sc0)),
                                                      qv, sa[e], 0, 0, 0);
      sa[2 + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, fp4x8_to_bf16x8(cd1[c][k], sc1)), qv, sa[2 + e], 0, 0, 0);
    }
  }
  const f32x4 s0 = sa[0] + sa[1], s1 = sa[2] + sa[3];
  float z[8];
  int rr[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rr[j] = base + ((j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool v0 = rr[j] < nrows && rowid[rr[j]] >= 0;
    const bool v1 = rr[4 + j] < nrows && rowid[rr[4 + j]] >= 0;
    z[j] = v0 ? s0[j] * scale_log2 : -INFINITY;
    z[4 + j] = v1 ? s1[j] * scale_log2 : -INFINITY;
  }
  bf16x8 pa_hi, pa_lo;
  softmax_tile(z, st, acc, pa_hi, pa_lo);
  // PV: lane (n, g) reads the 16-byte MX block n of its 8 rows.
  u32x4 cd[8];
  float sc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint8_t* rp = rows + rr[j] * kRowB;
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

// One 32-row tile of window rows, read from global memory.
__device__ __forceinline__ void win_tile(const DecArgs& a, int b, int t, int base, const uint16_t* qs, Softmax& st,
                                         f32x4 (&acc)[32]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, g = lane >> 4;
  const int64_t qr0 = win_row(a, b, t, base + n), qr1 = win_row(a, b, t, base + 16 + n);
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* qrow = qs + n * kQStride + 128 * g;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 r0[8], r1[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int dim = 128 * g + 8 * (8 * half + s);
      r0[s] = qr0 >= 0 ? *reinterpret_cast<const u32x4*>(a.swa + qr0 * CSA2_D_LATENT + dim) : u32x4{0u, 0u, 0u, 0u};
      r1[s] = qr1 >= 0 ? *reinterpret_cast<const u32x4*>(a.swa + qr1 * CSA2_D_LATENT + dim) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 8 * (8 * half + s)));
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r0[s]), qv, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r1[s]), qv, s1, 0, 0, 0);
    }
  }
  int64_t pv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = win_row(a, b, t, base + ((j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4)));
  float z[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    z[j] = pv[j] >= 0 ? s0[j] * a.scale_log2 : -INFINITY;
    z[4 + j] = pv[4 + j] >= 0 ? s1[j] * a.scale_log2 : -INFINITY;
  }
  bf16x8 pa_hi, pa_lo;
  softmax_tile(z, st, acc, pa_hi, pa_lo);
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {   // dims 32n + 8ch .. +7
    u32x4 rv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rv[j] = pv[j] >= 0 ? *reinterpret_cast<const u32x4*>(a.swa + pv[j] * CSA2_D_LATENT + 32 * n + 8 * ch)
                         : u32x4{0u, 0u, 0u, 0u};
    uint32_t d[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int j = 0; j < 8; ++j) d[k][j] = rv[j][k];
    }
    pv_quad(acc, 8 * ch, pa_hi, pa_lo, d);
  }
}

__global__ __launch_bounds__(kThreads) void sparse_decode_kernel(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t* rows = lds + kOffRows;
  uint16_t* qs = reinterpret_cast<uint16_t*>(lds + kOffQ);
  int32_t* rowid = reinterpret_cast<int32_t*>(lds + kOffRowId);
  float* m_w = reinterpret_cast<float*>(lds + kOffSm);
  float* l_w = m_w + kWaves * 16;
  float* m_g = l_w + kWaves * 16;
  float* l_g = m_g + 16;

  // XCD-aware mapping: consecutive workgroup ids go to different XCDs, so all head
  // groups of a sequence get the same id modulo 8.
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int b = xcd + 8 * (li / a.HG);
  const int hg = li % a.HG;
  if (b >= a.B) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, g = lane >> 4;

  int64_t L = a.ctx_len[b];
  if (L < 0) L = 0;
  const int n_vis = (int)(L >> 1);
  const int t = (int)L - 1;

  for (int i = tid; i < 16 * 64; i += kThreads) {
    const int h = i >> 6, c = i & 63;
    *reinterpret_cast<u32x4*>(qs + h * kQStride + 8 * c) =
        *reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.H + hg * 16 + h) * CSA2_D_LATENT + 8 * c);
  }

  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  Softmax st{-INFINITY, 0.f};

  const int n_batches = a.topk > 0 ? (a.topk + kBatchRows - 1) / kBatchRows : 1;
  const int n_win_tiles = (a.W + 31) >> 5;
  for (int bt = 0; bt < n_batches; ++bt) {
    const int r0 = bt * kBatchRows;
    const int nrows = max(0, min(a.topk - r0, kBatchRows));
    for (int i = tid; i < nrows; i += kThreads) rowid[i] = fp4_row_id(a, b, n_vis, r0 + i);
    __syncthreads();
    // stage the batch: LDS chunk c (16 bytes) = piece c%17 of row c/17
    const int chunks = nrows * 17;
    const int n_ins = (chunks + 63) >> 6;
    for (int ins = wid; ins < n_ins; ins += kWaves) {
      const int c = ins * 64 + lane;
      if (c < chunks) {
        const int r = c / 17, piece = c - r * 17;
        const int rid = rowid[r];
        if (rid >= 0) {
          const uint8_t* src = piece < 16 ? a.lat_codes + (int64_t)rid * CSA2_LAT_CODE_BYTES + 16 * piece
                                          : a.lat_scales + (int64_t)rid * CSA2_LAT_SCALE_BYTES;
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), rows + ins * 1024, 16, 0, 0);
        }
      }
    }
    // window tiles overlap the copies (first batch only), taken by the last waves
    if (bt == 0) {
      for (int wt = kWaves - 1 - wid; wt < n_win_tiles; wt += kWaves) win_tile(a, b, t, wt * 32, qs, st, acc);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // absent rows and the tail of the last tile hold stale bytes: zero them
    const int padded = ((nrows + 31) >> 5) << 5;
    for (int c = tid; c < padded * 17; c += kThreads) {
      const int r = c / 17;
      if (r >= nrows || rowid[r] < 0) *reinterpret_cast<u32x4*>(rows + c * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    for (int tile = wid; tile * 32 < nrows; tile += kWaves)
      fp4_tile(rows, rowid, nrows, tile * 32, qs, a.scale_log2, st, acc);
    __syncthreads();
  }

  // ---------------- merge the waves ----------------
  float l_head = st.l_part;
  l_head += __shfl_xor(l_head, 16, kWave);
  l_head += __shfl_xor(l_head, 32, kWave);
  if (g == 0) {
    m_w[wid * 16 + n] = st.m_run;
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
    const float mh = __shfl(st.m_run, 4 * g + i, kWave);
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
    *reinterpret_cast<u32x2*>(a.out + ((int64_t)b * a.H + hg * 16 + h) * CSA2_D_LATENT + d) =
        u32x2{v0 | (v1 << 16), v2 | (v3 << 16)};
  }
  if (a.lse && tid < 16) {
    const float l = l_g[tid];
    a.lse[(int64_t)b * a.H + hg * 16 + tid] = l > 0.f ? (m_g[tid] + log2f(l)) * kLn2 : -INFINITY;
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

int launch_sparse_decode(const csa2_cache_t& c, int B, int H, const int32_t* ctx_len,
                         const uint16_t* q, const int32_t* topk_idx, int topk, const uint16_t* swa,
                         int W, float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t s) {
  (void)ws;
  if (!lds_limit_set()) return CSA2_EHIP;
  DecArgs a;
  a.lat_codes = c.lat_codes;
  a.lat_scales = c.lat_scales;
  a.block_table = c.block_table;
  a.n_pages = c.n_pages;
  a.max_pages = c.max_pages;
  a.ctx_len = ctx_len;
  a.q = q;
  a.topk_idx = topk_idx;
  a.topk = topk;
  a.swa = swa;
  a.W = W;
  a.scale_log2 = sm_scale * kLog2e;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.HG = H / 16;
  const int64_t grid = 8 * ((int64_t)(B + 7) / 8) * a.HG;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  hipLaunchKernelGGL(sparse_decode_kernel, dim3((unsigned)grid), dim3(kThreads), kLdsBytes, s, a);
  return hip_status();
}

}  // namespace csa2
