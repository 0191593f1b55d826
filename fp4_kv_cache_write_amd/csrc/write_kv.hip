// Write path: pairwise merge of two tokens into one entry (ratio 2) or one token per
// entry (ratio 1), MXFP4 quantisation of the 512-d latent and the 64-d indexer key,
// scatter into the paged cache.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §1.1 (the encoder
// merges two adjacent positions with learned per-channel weights) and §2.3.1 (no
// window overlap, no absolute position embedding; the indexer key is derived from
// the entry; the ratio-1 special case leaves the decoder's entries unmerged).  FP4
// block format and rounding: see csa2.h.
//
// One wavefront per entry.  Lane l owns channels 8l..8l+7: four 16-byte loads
// (x and w of both tokens), one fused multiply-add per channel, an MX block of 32
// channels spans 4 adjacent lanes (max via two DPP quad permutations), four hardware
// converts make the lane's 8 codes, and the lane stores one dword of codes, so a wave
// writes the entry's 256 code bytes in one coalesced store.  The kernel is HBM-bound:
// 4 KB read and 306 B written per entry.
#include <algorithm>

#include "common.h"
#include "entry_write.h"
#include "internal.h"

namespace csa2 {
namespace {

// The wave index is made uniform, so the entry, its sequence and the page lookup are
// scalar: start_tok and the block table come through scalar loads, which do not wait
// behind the entry's vector loads.  A wave past the end repeats the last entry's loads
// and stores nothing, so no branch sits between the kernel-argument loads.
__global__ __launch_bounds__(256) void write_kv_kernel(WriteArgs a, int total) {
  const int e0 = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool live = e0 < total;
  const uint32_t e = (uint32_t)(live ? e0 : total - 1);
  const uint32_t b = e / (uint32_t)a.half;
  write_entry_wave(a, (int)b, (int)(e - b * (uint32_t)a.half), threadIdx.x & 63, live);
}


// Write with the indexer key projected from the entry ([P1] §2.3.1: the indexer key
// is a projection of the compressed entry; the weights are the caller's).  The key
// is k_o = fp32(s_512), s_{d+1} = fp64(s_d + P[o][d] * y[d]) over channels d = 0..511
// in order: a bf16 x fp32 product has at most 32 significant bits, so each fma below
// rounds exactly where that sum does, and the bytes match a plain evaluation of it.
//
// The 64 KB weight matrix is staged transposed in LDS once per workgroup (pt[d][o]),
// and each wave takes groups of 8 entries in a grid-stride loop.  The wave merges and
// stores the 8 latents one by one as write_kv_kernel does and parks their y in padded
// LDS rows; then lane (e, g) = (lane / 8, lane % 8) runs the 8 chains of outputs
// 8g..8g+7 of entry e side by side -- one 16-byte weight read and one y value per
// channel feed 8 independent fmas -- and those 8 outputs are exactly the channels the
// MX quantiser expects in that lane, so the key is quantised and stored in place.
constexpr int kProjWaves = 4;
constexpr int kProjEntries = 8;                                  // entries per wave pass
constexpr int kProjYPitch = CSA2_D_LATENT + 4;                   // floats per y row (bank offset 4)
constexpr size_t kProjLds = (size_t)CSA2_D_LATENT * CSA2_D_INDEX * 2 +
                            (size_t)kProjWaves * kProjEntries * kProjYPitch * 4;

__global__ __launch_bounds__(256) void write_kv_proj_kernel(
    uint8_t* __restrict__ lat_codes, uint8_t* __restrict__ lat_scales,
    uint8_t* __restrict__ idx_codes, uint8_t* __restrict__ idx_scales, int n_pages,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ start_tok,
    int half, int64_t total, const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ w_proj, int ratio) {
  extern __shared__ __attribute__((aligned(16))) uint32_t plds[];
  uint16_t* pt = reinterpret_cast<uint16_t*>(plds);               // [512][64]: pt[d*64 + o] = P[o][d]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  float* ys = reinterpret_cast<float*>(plds + CSA2_D_LATENT * CSA2_D_INDEX / 2) + wid * kProjEntries * kProjYPitch;
  // staging: thread (o = t % 64, channels 8c..8c+7) reads 16 bytes of row o and writes
  // 8 weights; the 64 lanes of a store write 64 adjacent weights
  for (int t = threadIdx.x; t < CSA2_D_INDEX * (CSA2_D_LATENT / 8); t += blockDim.x) {
    const int o = t & (CSA2_D_INDEX - 1), c = t / CSA2_D_INDEX;
    const u32x4 v = *reinterpret_cast<const u32x4*>(w_proj + o * CSA2_D_LATENT + 8 * c);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      pt[(8 * c + 2 * q) * CSA2_D_INDEX + o] = (uint16_t)(v[q] & 0xffffu);
      pt[(8 * c + 2 * q + 1) * CSA2_D_INDEX + o] = (uint16_t)(v[q] >> 16);
    }
  }
  __syncthreads();
  // cache row of entry e, or -1 (past the end, bad start, absent page)
  auto entry_row = [&](int64_t e, int& b, int& i) -> int64_t {
    if (e >= total) return -1;
    b = (int)(e / half);
    i = (int)(e - (int64_t)b * half);
    const int st = start_tok[b];
    if (st < 0 || (ratio == 2 && (st & 1))) return -1;           // caller contract: even start at ratio 2
    const int j = (ratio == 2 ? (st >> 1) : st) + i;
    const int page = page_of(block_table, max_pages, n_pages, b, j);
    return page < 0 ? -1 : (int64_t)page * CSA2_PAGE + (j & (CSA2_PAGE - 1));
  };
  const int es = lane >> 3, og = lane & 7;
  const int64_t n_groups = (total + kProjEntries - 1) / kProjEntries;
  for (int64_t gi = (int64_t)blockIdx.x * kProjWaves + wid; gi < n_groups; gi += (int64_t)gridDim.x * kProjWaves) {
    for (int q = 0; q < kProjEntries; ++q) {                      // latents, one entry at a time
      int b = 0, i = 0;
      const int64_t row = entry_row(gi * kProjEntries + q, b, i);   // wave-uniform
      float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (row >= 0) entry_latent(x, w, b, i, half, ratio, lane, y);
      uint32_t codes, u;
      mx_quant8(y, codes, u);
      if (row >= 0) {
        *reinterpret_cast<uint32_t*>(lat_codes + row * CSA2_LAT_CODE_BYTES + lane * 4) = codes;
        if ((lane & 3) == 0) lat_scales[row * CSA2_LAT_SCALE_BYTES + (lane >> 2)] = (uint8_t)u;
      }
      float* yr = ys + q * kProjYPitch + lane * 8;
      *reinterpret_cast<f32x4*>(yr) = f32x4{y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4*>(yr + 4) = f32x4{y[4], y[5], y[6], y[7]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");            // the 8 y rows are in LDS
    double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    const float* yrow = ys + es * kProjYPitch;
    const uint16_t* pcol = pt + og * 8;
#pragma unroll 2
    for (int d = 0; d < CSA2_D_LATENT; d += 4) {
      const f32x4 yv = *reinterpret_cast<const f32x4*>(yrow + d);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const u32x4 pv = *reinterpret_cast<const u32x4*>(pcol + (d + dd) * CSA2_D_INDEX);
        const double yd = (double)yv[dd];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[2 * r] = fma((double)lo_bf16(pv[r]), yd, acc[2 * r]);
          acc[2 * r + 1] = fma((double)hi_bf16(pv[r]), yd, acc[2 * r + 1]);
        }
      }
    }
    float kv[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) kv[r] = (float)acc[r];
    uint32_t codes, u;
    mx_quant8(kv, codes, u);                                      // block = lanes 8e..8e+3 / 8e+4..8e+7
    int b = 0, i = 0;
    const int64_t row = entry_row(gi * kProjEntries + es, b, i);
    if (row >= 0) {
      *reinterpret_cast<uint32_t*>(idx_codes + row * CSA2_IDX_CODE_BYTES + og * 4) = codes;
      if ((og & 3) == 0) idx_scales[row * CSA2_IDX_SCALE_BYTES + (og >> 2)] = (uint8_t)u;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");            // y rows free for the next group
  }
}

// HISA block summaries ([P1] §2.3.4, HISA): block k of a sequence covers entries
// k*cb .. k*cb+cb-1; its summary is the mean of the dequantised indexer keys of the
// entries that are visible and present, summed in float32 in entry order and divided
// once by their count (zero key for an empty block), stored as an MXFP4 indexer key
// in slot k of the block-key cache.  One wave per (sequence, block): lane l sums
// dimension l (each e2m1 x 2^(u-127) term is exact in float32); the 64 means are
// regrouped through LDS so that lanes 0..7 quantise 8 each, as for any key.
__device__ __forceinline__ float e2m1_times_scale(uint32_t c, uint32_t u) {
  const uint32_t eb = (c >> 1) & 3u, mb = c & 1u;
  const float mag = eb == 0u ? 0.5f * (float)mb : ldexpf(1.0f + 0.5f * (float)mb, (int)eb - 1);
  const float v = ldexpf(mag, (int)u - 127);                     // exact: at most 2 significant bits
  return (c & 8u) ? -v : v;
}

__global__ __launch_bounds__(256) void block_keys_kernel(
    const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales, int n_pages,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ ctx_len, int64_t max_ctx,
    int vshift, int cb_shift, const int32_t* __restrict__ blk_first, int n_span, int B,
    uint8_t* __restrict__ bk_codes, uint8_t* __restrict__ bk_scales, int bk_n_pages,
    const int32_t* __restrict__ bk_table, int bk_max_pages, int32_t* __restrict__ n_blocks_out) {
  __shared__ float means[4][CSA2_D_INDEX];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t wv = (int64_t)blockIdx.x * 4 + wid;
  if (wv >= (int64_t)B * n_span) return;                         // whole wave
  const int b = (int)(wv / n_span);
  const int r = (int)(wv - (int64_t)b * n_span);
  int64_t L = ctx_len[b];
  L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int n_vis = (int)(L >> vshift);
  const int cb = 1 << cb_shift;
  const int nb = (n_vis + cb - 1) >> cb_shift;
  if (r == 0 && n_blocks_out && lane == 0) n_blocks_out[b] = nb;
  const int first = blk_first ? max(blk_first[b], 0) : 0;
  const int k = first + r;
  if (k >= nb) return;
  const int j0 = k << cb_shift;
  const int page = page_of(block_table, max_pages, n_pages, b, j0);   // cb divides 64: one page per block
  float sum = 0.0f;
  int cnt = 0;
  if (page >= 0) {
    for (int i = 0; i < cb && j0 + i < n_vis; ++i) {
      const int64_t row = (int64_t)page * CSA2_PAGE + ((j0 + i) & (CSA2_PAGE - 1));
      const uint32_t byte = idx_codes[row * CSA2_IDX_CODE_BYTES + (lane >> 1)];
      const uint32_t u = idx_scales[row * CSA2_IDX_SCALE_BYTES + (lane >> 5)];
      sum += e2m1_times_scale((byte >> (4 * (lane & 1))) & 15u, u);
      ++cnt;
    }
  }
  means[wid][lane] = cnt > 0 ? __fdiv_rn(sum, (float)cnt) : 0.0f;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");            // the wave's 64 means are in LDS
  float kv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) kv[q] = lane < 8 ? means[wid][lane * 8 + q] : 0.0f;
  uint32_t codes, u;
  mx_quant8(kv, codes, u);
  const int bpage = page_of(bk_table, bk_max_pages, bk_n_pages, b, k);
  if (lane < 8 && bpage >= 0) {
    const int64_t brow = (int64_t)bpage * CSA2_PAGE + (k & (CSA2_PAGE - 1));
    *reinterpret_cast<uint32_t*>(bk_codes + brow * CSA2_IDX_CODE_BYTES + lane * 4) = codes;
    if ((lane & 3) == 0) bk_scales[brow * CSA2_IDX_SCALE_BYTES + (lane >> 2)] = (uint8_t)u;
  }
}

// Dequantise entries through the page table with the kernels' own FP4 decode.
__global__ __launch_bounds__(256) void debug_gather_kernel(
    const uint8_t* __restrict__ lat_codes, const uint8_t* __restrict__ lat_scales,
    const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales, int n_pages,
    const int32_t* __restrict__ block_table, int max_pages, const int32_t* __restrict__ idx, int n,
    int64_t total, float* __restrict__ out_lat, float* __restrict__ out_idx) {
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= total) return;
  const int lane = threadIdx.x & 63;
  const int b = (int)(e / n);
  const int j = idx[e];
  const int page = page_of(block_table, max_pages, n_pages, b, j);
  const float nan = __uint_as_float(0x7fc00000u);
  const int64_t row = (int64_t)page * CSA2_PAGE + (j & (CSA2_PAGE - 1));
  if (out_lat) {
    float* o = out_lat + e * CSA2_D_LATENT + lane * 8;
    if (page < 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = nan;
    } else {
      const uint32_t codes =
          *reinterpret_cast<const uint32_t*>(lat_codes + row * CSA2_LAT_CODE_BYTES + lane * 4);
      const float sc = e8m0_scale(lat_scales[row * CSA2_LAT_SCALE_BYTES + (lane >> 2)]);
      const u32x4 v = fp4x8_to_bf16x8(codes, sc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[2 * q] = lo_bf16(v[q]);
        o[2 * q + 1] = hi_bf16(v[q]);
      }
    }
  }
  if (out_idx && lane < 8) {
    float* o = out_idx + e * CSA2_D_INDEX + lane * 8;
    if (page < 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = nan;
    } else {
      const uint32_t codes =
          *reinterpret_cast<const uint32_t*>(idx_codes + row * CSA2_IDX_CODE_BYTES + lane * 4);
      const float sc = e8m0_scale(idx_scales[row * CSA2_IDX_SCALE_BYTES + (lane >> 2)]);
      const u32x4 v = fp4x8_to_bf16x8(codes, sc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[2 * q] = lo_bf16(v[q]);
        o[2 * q + 1] = hi_bf16(v[q]);
      }
    }
  }
}

}  // namespace

int launch_write_kv(const csa2_cache_t& c, int B, const int32_t* start_tok, int T_new,
                    const uint16_t* x, const uint16_t* w, const uint16_t* k_idx, hipStream_t s) {
  const int ratio = cache_ratio(c);
  const int half = T_new / ratio;   // entries per sequence
  const int64_t total = (int64_t)B * half;
  if (total == 0) return CSA2_OK;
  if (total > 0x7fffffff) return CSA2_EUNSUPPORTED;
  const int64_t grid = (total + 3) / 4;
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     write_args(c, start_tok, half, x, w, k_idx, ratio), (int)total);
  return hip_status();
}

int launch_write_kv_proj(const csa2_cache_t& c, int B, const int32_t* start_tok, int T_new,
                         const uint16_t* x, const uint16_t* w, const uint16_t* w_proj, hipStream_t s) {
  static const bool lds_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(write_kv_proj_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)kProjLds) == hipSuccess;
  if (!lds_ok) return CSA2_EHIP;
  const int ratio = cache_ratio(c);
  const int half = T_new / ratio;   // entries per sequence
  const int64_t total = (int64_t)B * half;
  if (total == 0) return CSA2_OK;
  // one workgroup per CU (129 KB of LDS); at most one group of 8 entries per wave
  const int64_t groups = (total + kProjEntries - 1) / kProjEntries;
  const int64_t grid = std::min<int64_t>((groups + kProjWaves - 1) / kProjWaves, 256);
  hipLaunchKernelGGL(write_kv_proj_kernel, dim3((unsigned)grid), dim3(64 * kProjWaves), kProjLds, s, c.lat_codes,
                     c.lat_scales, c.idx_codes, c.idx_scales, c.n_pages, c.block_table,
                     c.max_pages, start_tok, half, total, x, w, w_proj, ratio);
  return hip_status();
}

int launch_block_keys(const csa2_cache_t& c, const csa2_cache_t& blocks, int B, const int32_t* ctx_len,
                      int64_t max_ctx, int cand_block, const int32_t* blk_first, int n_span, int32_t* n_blocks_out,
                      hipStream_t s) {
  const int cb_shift = __builtin_ctz((unsigned)cand_block);
  if (blk_first == nullptr) n_span = (int)(((max_ctx >> vis_shift(c)) + cand_block - 1) >> cb_shift);
  const int64_t waves = (int64_t)B * n_span;
  if (waves == 0) return CSA2_OK;
  const int64_t grid = (waves + 3) / 4;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  hipLaunchKernelGGL(block_keys_kernel, dim3((unsigned)grid), dim3(256), 0, s, c.idx_codes, c.idx_scales, c.n_pages,
                     c.block_table, c.max_pages, ctx_len, max_ctx, vis_shift(c), cb_shift, blk_first, n_span, B,
                     blocks.idx_codes, blocks.idx_scales, blocks.n_pages, blocks.block_table, blocks.max_pages,
                     n_blocks_out);
  return hip_status();
}

int launch_debug_gather(const csa2_cache_t& c, int B, const int32_t* idx, int n, float* out_lat,
                        float* out_idx, hipStream_t s) {
  const int64_t total = (int64_t)B * n;
  if (total == 0) return CSA2_OK;
  const int64_t grid = (total + 3) / 4;
  if (grid > 0x7fffffff) return CSA2_EUNSUPPORTED;
  hipLaunchKernelGGL(debug_gather_kernel, dim3((unsigned)grid), dim3(256), 0, s, c.lat_codes,
                     c.lat_scales, c.idx_codes, c.idx_scales, c.n_pages, c.block_table,
                     c.max_pages, idx, n, total, out_lat, out_idx);
  return hip_status();
}

}  // namespace csa2
