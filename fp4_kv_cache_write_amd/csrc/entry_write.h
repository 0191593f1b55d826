// One entry of the write path, done by one wavefront: used by the write kernel and
// by the Full scan when it performs the step's write itself.
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §1.1 (the encoder
// merges two adjacent positions with learned per-channel weights) and §2.3.1 (no
// window overlap, no absolute position embedding; the indexer key is derived from
// the entry; the ratio-1 special case leaves the decoder's entries unmerged).  FP4
// block format and rounding: see csa2.h.
#pragma once

#include "common.h"

namespace csa2 {

// Quantise the lane's 8 values; the 32-value block is lanes 4q..4q+3.  The block
// maximum is reduced over the quad with two DPP quad permutations.  The codes come
// from the gfx950 convert v_cvt_scalef32_pk_fp4_f32, which divides by the power of
// two held in its scale operand's exponent field and rounds to the nearest e2m1 value
// with ties to the even code, saturating at 6 (sign kept, -0 -> code 8).  Measured on
// the MI355X against that rule: every value of a dense sweep of [0, 9) and of its
// negatives, the ties and their neighbours, at scale exponent fields 0..254,
// subnormal inputs included -- no difference.  So the codes are those of the plain
// rule of csa2_write_kv; only non-finite inputs (outside that rule) differ from it.
__device__ __forceinline__ void mx_quant8(const float (&y)[8], uint32_t& codes, uint32_t& u) {
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(y[k]));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xb1, 0xf, 0xf, false)));  // quad_perm 1,0,3,2
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4e, 0xf, 0xf, false)));  // quad_perm 2,3,0,1
  // scale exponent e = floor(log2 a) - 2 clamped at -127  ->  byte u = e + 127
  const uint32_t bexp = (__float_as_uint(a) >> 23) & 0xffu;
  u = bexp > 2u ? bexp - 2u : 0u;
  const float sc = __uint_as_float(u << 23);   // exponent field u: the scale 2^e
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], sc, 0);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[2], y[3], sc, 1);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[4], y[5], sc, 2);
  c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, y[6], y[7], sc, 3);
  codes = a == 0.0f ? 0u : c;   // an all-zero block stores +0 codes
}

__device__ __forceinline__ float lo_bf16(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// Channels 8l..8l+7 (lane l) of entry i of sequence b before quantisation: the fp32
// merge of its two tokens (ratio 2) or the token itself (ratio 1).  The raw bf16 words
// are loaded first (entry_words) and combined later (latent_of), so a caller can issue
// the loads before work that does not depend on them.
struct EntryWords {
  u32x4 xa, xb, wa, wb;   // ratio 1: xa only
};

__device__ __forceinline__ void entry_words(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int b,
                                            int i, int half, int ratio, int lane, EntryWords& t) {
  if (ratio == 2) {
    const int64_t tok0 = ((int64_t)b * 2 * half + 2 * i) * CSA2_D_LATENT + lane * 8;
    t.xa = *reinterpret_cast<const u32x4*>(x + tok0);
    t.xb = *reinterpret_cast<const u32x4*>(x + tok0 + CSA2_D_LATENT);
    t.wa = *reinterpret_cast<const u32x4*>(w + tok0);
    t.wb = *reinterpret_cast<const u32x4*>(w + tok0 + CSA2_D_LATENT);
  } else {
    t.xa = *reinterpret_cast<const u32x4*>(x + ((int64_t)b * half + i) * CSA2_D_LATENT + lane * 8);
  }
}

__device__ __forceinline__ void latent_of(const EntryWords& t, int ratio, float (&y)[8]) {
  if (ratio == 2) {
    // y = w0*x0 + w1*x1 with one rounding (w1*x1 is exact in fp32)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] = fmaf(lo_bf16(t.wa[q]), lo_bf16(t.xa[q]), lo_bf16(t.wb[q]) * lo_bf16(t.xb[q]));
      y[2 * q + 1] = fmaf(hi_bf16(t.wa[q]), hi_bf16(t.xa[q]), hi_bf16(t.wb[q]) * hi_bf16(t.xb[q]));
    }
  } else {
    // the token itself (bf16 is exact in fp32)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] = lo_bf16(t.xa[q]);
      y[2 * q + 1] = hi_bf16(t.xa[q]);
    }
  }
}

__device__ __forceinline__ void entry_latent(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int b,
                                             int i, int half, int ratio, int lane, float (&y)[8]) {
  EntryWords t;
  entry_words(x, w, b, i, half, ratio, lane, t);
  latent_of(t, ratio, y);
}

// The step's write: half entries per sequence from start_tok[b] (a token position;
// entry start_tok[b] / ratio), inputs [B][half * ratio][512] (x, w) and [B][half][64].
struct WriteArgs {
  uint8_t* lat_codes;
  uint8_t* lat_scales;
  uint8_t* idx_codes;
  uint8_t* idx_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* start_tok;
  int half, ratio;
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* k_idx;
};

inline WriteArgs write_args(const csa2_cache_t& c, const int32_t* start_tok, int half, const uint16_t* x,
                            const uint16_t* w, const uint16_t* k_idx, int ratio) {
  return WriteArgs{c.lat_codes, c.lat_scales, c.idx_codes, c.idx_scales, c.block_table, c.n_pages, c.max_pages,
                   start_tok, half, ratio, x, w, k_idx};
}

// First entry of sequence b's write, or -1 when its start breaks the contract (negative,
// or odd at ratio 2) and nothing is written.
__device__ __forceinline__ int write_first_entry(const WriteArgs& a, int b) {
  const int st = a.start_tok[b];
  if (st < 0 || (a.ratio == 2 && (st & 1))) return -1;
  return a.ratio == 2 ? (st >> 1) : st;
}

// Lane l of one wave: channels 8l..8l+7 of the latent of the write's entry i of
// sequence b and, in lanes 0..7, channels 8l..8l+7 of its indexer key; both are
// quantised and stored at the entry's cache row (nothing when its page is absent).
// Lane l stores one dword of latent codes, so the wave writes the entry's 256 code
// bytes in one coalesced store.
__device__ __forceinline__ void write_entry_wave(const WriteArgs& a, int b, int i, int lane, bool live = true) {
  // The entry's inputs do not depend on where it is stored: their loads are issued
  // first and are in flight during the page lookup (start_tok, then the block table).
  EntryWords t;
  entry_words(a.x, a.w, b, i, a.half, a.ratio, lane, t);
  u32x4 ka = u32x4{0u, 0u, 0u, 0u};   // lanes 0..7: channels 8l..8l+7 of the indexer key
  if (lane < 8) ka = *reinterpret_cast<const u32x4*>(a.k_idx + ((int64_t)b * a.half + i) * CSA2_D_INDEX + lane * 8);
  const int j0 = write_first_entry(a, b);
  if (j0 < 0 || !live) return;
  const int j = j0 + i;
  const int page = page_of(a.block_table, a.max_pages, a.n_pages, b, j);
  if (page < 0) return;
  const int64_t row = (int64_t)page * CSA2_PAGE + (j & (CSA2_PAGE - 1));

  float y[8];
  latent_of(t, a.ratio, y);
  uint32_t codes, u;
  mx_quant8(y, codes, u);
  *reinterpret_cast<uint32_t*>(a.lat_codes + row * CSA2_LAT_CODE_BYTES + lane * 4) = codes;
  if ((lane & 3) == 0) a.lat_scales[row * CSA2_LAT_SCALE_BYTES + (lane >> 2)] = (uint8_t)u;

  // ---- indexer key: lanes 0..7 own 8 channels each (two MX blocks) ----
  float kv[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {   // lanes 8..63 hold zeros
    kv[2 * q] = lo_bf16(ka[q]);
    kv[2 * q + 1] = hi_bf16(ka[q]);
  }
  mx_quant8(kv, codes, u);
  if (lane < 8) {
    *reinterpret_cast<uint32_t*>(a.idx_codes + row * CSA2_IDX_CODE_BYTES + lane * 4) = codes;
    if ((lane & 3) == 0) a.idx_scales[row * CSA2_IDX_SCALE_BYTES + (lane >> 2)] = (uint8_t)u;
  }
}

}  // namespace csa2
