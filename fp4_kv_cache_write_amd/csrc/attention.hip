// Sparse gather-attention for one decode query per sequence: the top-K FP4 latent
// rows plus the bf16 sliding window, one softmax, K = V = the 512-d latent.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §1.2 (window 128,
// every head shares one 512-d latent) and §2.3.1 (each query attends to the selected
// entries and the layer's window KV together); [P3] "DeepSeek V4.1 Flash
// architecture..." (scores -> weights summing to 1 -> weighted sum of values).
//
// Decomposition: one workgroup per (sequence, group of 16 heads); blockIdx is
// mapped so that the head groups of one sequence run on the same XCD and share its
// L2 for the gathered rows.  The rows are cut into 32-row tiles dealt round-robin to
// the 4 waves; each wave keeps its own online-softmax state and a 16 x 512 fp32
// output accumulator, and the waves are merged through LDS at the end.
//
// Per 32-row tile a wave runs:
//   QK  D[row][head] via 16x16x32 bf16 MFMA; A = rows (lane: row l%16, dims
//       128g+8s..+7 at k-step s, g = l/16), B = q (lane: head l%16, same dims).
//       FP4 rows are turned into bf16 operands by the hardware convert with the
//       e8m0 scale folded in (exact).
//   softmax  the lane then holds rows {4g..4g+3, 16+4g..16+4g+3} of head l%16 --
//       exactly the K-slots of the P operand of the next MFMA, so P needs no
//       cross-lane movement.  The running maximum is only raised when a tile
//       exceeds it by 2^8, which bounds p by 256 and saves rescaling the
//       accumulators on almost every tile; the result is exact either way.
//   PV  O[head][dim] += P . R via 16x16x32 bf16 MFMA, n-tile t holding dims 32n+t
//       for lane column n, so each lane loads one contiguous 16-byte MX block per
//       row and transposes register pairs into the B operand.  P is split into a
//       bf16 head and a bf16 residual (two MFMAs) so the weights enter with ~16
//       bits instead of 8.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;   // log2 headroom before the running max is raised

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

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Row of tile-local index r: byte offset of its latent codes (FP4 tile) or of its
// bf16 row (window tile); -1 when the row is absent.
__device__ __forceinline__ int64_t fp4_row(const DecArgs& a, int b, int n_vis, int i) {
  if (i >= a.topk) return -1;
  const int e = a.topk_idx[(int64_t)b * a.topk + i];
  if (e < 0 || e >= n_vis) return -1;
  const int page = page_of(a.block_table, a.max_pages, a.n_pages, b, e);
  if (page < 0) return -1;
  return (int64_t)page * CSA2_PAGE + (e & (CSA2_PAGE - 1));
}

__device__ __forceinline__ int64_t win_row(const DecArgs& a, int b, int t, int w) {
  if (w >= a.W) return -1;
  const int pos = t - (a.W - 1) + w;
  if (pos < 0) return -1;
  return (int64_t)b * a.W + (pos % a.W);
}

__global__ __launch_bounds__(kThreads) void sparse_decode_kernel(DecArgs a) {
  __shared__ float o_sum[16 * CSA2_D_LATENT];
  __shared__ float m_w[kWaves][16];
  __shared__ float l_w[kWaves][16];
  __shared__ float m_g[16];
  __shared__ float l_g[16];

  // XCD-aware mapping: consecutive workgroup ids go to different XCDs, so give
  // all head groups of a sequence the same id modulo 8.
  const int xcd = blockIdx.x & 7;
  const int li = blockIdx.x >> 3;
  const int b = xcd + 8 * (li / a.HG);
  const int hg = li % a.HG;
  if (b >= a.B) return;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = lane & 15, g = lane >> 4;

  for (int i = tid; i < 16 * CSA2_D_LATENT; i += kThreads) o_sum[i] = 0.f;

  int64_t L = a.ctx_len[b];
  if (L < 0) L = 0;
  const int n_vis = (int)(L >> 1);
  const int t = (int)L - 1;

  // q operand: head hg*16+n, dims 128g + 8s .. +7 for k-step s (16 x 16 bytes)
  u32x4 qf[16];
  {
    const uint16_t* qp = a.q + ((int64_t)b * a.H + hg * 16 + n) * CSA2_D_LATENT + 128 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qp + 8 * s);
  }

  f32x4 acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max (log2 units) for head n
  float l_part = 0.f;        // this lane's share of the softmax denominator

  const int n_fp4 = (a.topk + 31) >> 5;
  const int n_win = (a.W + 31) >> 5;
  const int n_tiles = n_fp4 + n_win;

  for (int tile = wid; tile < n_tiles; tile += kWaves) {
    const bool is_fp4 = tile < n_fp4;
    const int base = (is_fp4 ? tile : tile - n_fp4) * 32;
    // rows this lane reads for QK (row-tiles 0,1 at row n) and for PV (slots j)
    int64_t qk_row[2], pv_row[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      qk_row[h] = is_fp4 ? fp4_row(a, b, n_vis, base + 16 * h + n) : win_row(a, b, t, base + 16 * h + n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
      pv_row[j] = is_fp4 ? fp4_row(a, b, n_vis, base + r) : win_row(a, b, t, base + r);
    }

    // ---------------- QK ----------------
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (is_fp4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 cd[4];
        uint32_t scb = 0u;
        if (qk_row[h] >= 0) {
          const uint8_t* cp = a.lat_codes + qk_row[h] * CSA2_LAT_CODE_BYTES + 64 * g;
#pragma unroll
          for (int c = 0; c < 4; ++c) cd[c] = *reinterpret_cast<const u32x4*>(cp + 16 * c);
          scb = *reinterpret_cast<const uint32_t*>(a.lat_scales + qk_row[h] * CSA2_LAT_SCALE_BYTES + 4 * g);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) cd[c] = u32x4{0u, 0u, 0u, 0u};
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float sc = e8m0_scale((scb >> (8 * c)) & 0xffu);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const u32x4 rf = fp4x8_to_bf16x8(cd[c][k], sc);
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rf),
                                                           __builtin_bit_cast(bf16x8, qf[4 * c + k]),
                                                           sacc, 0, 0, 0);
          }
        }
        if (h == 0) s0 = sacc; else s1 = sacc;
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* rp = a.swa + (qk_row[h] >= 0 ? qk_row[h] : 0) * CSA2_D_LATENT + 128 * g;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          u32x4 rf = u32x4{0u, 0u, 0u, 0u};
          if (qk_row[h] >= 0) rf = *reinterpret_cast<const u32x4*>(rp + 8 * s);
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, rf),
                                                         __builtin_bit_cast(bf16x8, qf[s]), sacc, 0, 0, 0);
        }
        if (h == 0) s0 = sacc; else s1 = sacc;
      }
    }

    // ---------------- softmax (head n; rows = the P operand's K-slots) ----------------
    float z[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      z[j] = pv_row[j] >= 0 ? s0[j] * a.scale_log2 : -INFINITY;
      z[4 + j] = pv_row[4 + j] >= 0 ? s1[j] * a.scale_log2 : -INFINITY;
    }
    float tmax = z[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, z[j]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    // Raise head n's running max when this tile beats it by more than 2^kLazy.  The
    // accumulators of output head h sit in lanes with 4g+i == h, so every lane
    // fetches the factors of its 4 output heads from the softmax lanes 4g+i.
    float fac = 1.f;
    if (tmax > m_run + kLazy || (m_run == -INFINITY && tmax > -INFINITY)) {
      fac = (m_run == -INFINITY) ? 0.f : exp2f(m_run - tmax);
      l_part *= fac;
      m_run = tmax;
    }
    {
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
    }
    const float mb = (m_run == -INFINITY) ? 0.f : m_run;
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
    const bf16x8 pa_hi = __builtin_bit_cast(bf16x8, u32x4{phi[0], phi[1], phi[2], phi[3]});
    const bf16x8 pa_lo = __builtin_bit_cast(bf16x8, u32x4{plo[0], plo[1], plo[2], plo[3]});

    // ---------------- PV ----------------
    if (is_fp4) {
      u32x4 cd[8];
      float sc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (pv_row[j] >= 0) {
          cd[j] = *reinterpret_cast<const u32x4*>(a.lat_codes + pv_row[j] * CSA2_LAT_CODE_BYTES + 16 * n);
          sc[j] = e8m0_scale(a.lat_scales[pv_row[j] * CSA2_LAT_SCALE_BYTES + n]);
        } else {
          cd[j] = u32x4{0u, 0u, 0u, 0u};
          sc[j] = 0.f;
        }
      }
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {        // dword of the 16-byte block
#pragma unroll
        for (int by = 0; by < 4; ++by) {      // byte -> dims 32n + 8qd + 2by, +1
          uint32_t d[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            switch (by) {
              case 0: d[j] = fp4x2_to_bf16x2<0>(cd[j][qd], sc[j]); break;
              case 1: d[j] = fp4x2_to_bf16x2<1>(cd[j][qd], sc[j]); break;
              case 2: d[j] = fp4x2_to_bf16x2<2>(cd[j][qd], sc[j]); break;
              default: d[j] = fp4x2_to_bf16x2<3>(cd[j][qd], sc[j]); break;
            }
          }
          const int t0 = 8 * qd + 2 * by;
          const bf16x8 b0 = __builtin_bit_cast(
              bf16x8, u32x4{pack_lo(d[0], d[1]), pack_lo(d[2], d[3]), pack_lo(d[4], d[5]), pack_lo(d[6], d[7])});
          const bf16x8 b1 = __builtin_bit_cast(
              bf16x8, u32x4{pack_hi(d[0], d[1]), pack_hi(d[2], d[3]), pack_hi(d[4], d[5]), pack_hi(d[6], d[7])});
          acc[t0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b0, acc[t0], 0, 0, 0);
          acc[t0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b0, acc[t0], 0, 0, 0);
          acc[t0 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b1, acc[t0 + 1], 0, 0, 0);
          acc[t0 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b1, acc[t0 + 1], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {        // dims 32n + 8ch .. +7
        u32x4 rv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          rv[j] = pv_row[j] >= 0
                      ? *reinterpret_cast<const u32x4*>(a.swa + pv_row[j] * CSA2_D_LATENT + 32 * n + 8 * ch)
                      : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {         // dims pair 2k, 2k+1 of the chunk
          const int t0 = 8 * ch + 2 * k;
          const bf16x8 b0 = __builtin_bit_cast(
              bf16x8, u32x4{pack_lo(rv[0][k], rv[1][k]), pack_lo(rv[2][k], rv[3][k]),
                            pack_lo(rv[4][k], rv[5][k]), pack_lo(rv[6][k], rv[7][k])});
          const bf16x8 b1 = __builtin_bit_cast(
              bf16x8, u32x4{pack_hi(rv[0][k], rv[1][k]), pack_hi(rv[2][k], rv[3][k]),
                            pack_hi(rv[4][k], rv[5][k]), pack_hi(rv[6][k], rv[7][k])});
          acc[t0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b0, acc[t0], 0, 0, 0);
          acc[t0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b0, acc[t0], 0, 0, 0);
          acc[t0 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, b1, acc[t0 + 1], 0, 0, 0);
          acc[t0 + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, b1, acc[t0 + 1], 0, 0, 0);
        }
      }
    }
  }

  // ---------------- merge the waves ----------------
  float l_head = l_part;
  l_head += __shfl_xor(l_head, 16, kWave);
  l_head += __shfl_xor(l_head, 32, kWave);
  if (g == 0) {
    m_w[wid][n] = m_run;
    l_w[wid][n] = l_head;
  }
  __syncthreads();
  if (tid < 16) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, m_w[w][tid]);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (m_w[w][tid] > -INFINITY) l += l_w[w][tid] * exp2f(m_w[w][tid] - m);
    m_g[tid] = m;
    l_g[tid] = l;
  }
  __syncthreads();
  // lane (n, g) holds O[head 4g+i][dim 32n+t] in acc[t][i]; the running max of
  // head 4g+i lives in lane 4g+i.
  float f[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mh = __shfl(m_run, 4 * g + i, kWave);
    f[i] = (mh == -INFINITY) ? 0.f : exp2f(mh - m_g[4 * g + i]);
  }
#pragma unroll
  for (int tt = 0; tt < 32; ++tt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(&o_sum[(4 * g + i) * CSA2_D_LATENT + 32 * n + tt], acc[tt][i] * f[i]);
  }
  __syncthreads();
  for (int i = tid; i < 16 * CSA2_D_LATENT / 2; i += kThreads) {
    const int h = (2 * i) / CSA2_D_LATENT, d = (2 * i) % CSA2_D_LATENT;
    const float l = l_g[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const uint32_t v0 = f32_to_bf16_rne(o_sum[h * CSA2_D_LATENT + d] * inv);
    const uint32_t v1 = f32_to_bf16_rne(o_sum[h * CSA2_D_LATENT + d + 1] * inv);
    *reinterpret_cast<uint32_t*>(a.out + ((int64_t)b * a.H + hg * 16 + h) * CSA2_D_LATENT + d) = v0 | (v1 << 16);
  }
  if (a.lse && tid < 16) {
    const float l = l_g[tid];
    a.lse[(int64_t)b * a.H + hg * 16 + tid] = l > 0.f ? (m_g[tid] + log2f(l)) * kLn2 : -INFINITY;
  }
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
  hipLaunchKernelGGL(sparse_decode_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hip_status();
}

}  // namespace csa2
