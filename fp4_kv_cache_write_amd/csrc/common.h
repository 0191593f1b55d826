// Device helpers shared by the CSA2 kernels (gfx950 only).
//
// FP4 format (see csa2.h): e2m1 codes, two per byte with the even channel in the
// low nibble, one e8m0 scale byte u per 32 channels standing for 2^(u-127).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2.h"

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round fp32 to bf16, nearest with ties to even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// Scale operand of the FP4 convert for an e8m0 byte u (scale 2^(u-127)).  The
// convert reads only the exponent field of its fp32 scale operand, exponent field 0
// standing for 2^-127 as in e8m0, so the byte shifted into that field is the scale:
// one shift, no special case for u = 0.  (Checked against the exact multiplier,
// 2^-127 being the subnormal 0x00400000, on all 256 scale bytes x 256 code bytes.)
// Only valid as the convert's operand, not as an arithmetic multiplier.
__device__ __forceinline__ float e8m0_scale(uint32_t u) {
  return __uint_as_float(u << 23);
}

// Two e2m1 codes (byte SEL of `codes`: low nibble -> element 0) times `scale`, as bf16.
// e2m1 * 2^k is exact in bf16 over the whole range the quantiser produces.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t codes, float scale) {
  bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL);
  return __builtin_bit_cast(uint32_t, v);
}

// Eight e2m1 codes (one dword, channels 8 apart in order) -> 8 bf16 packed as 4 dwords.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t codes, float scale) {
  u32x4 r;
  r.x = fp4x2_to_bf16x2<0>(codes, scale);
  r.y = fp4x2_to_bf16x2<1>(codes, scale);
  r.z = fp4x2_to_bf16x2<2>(codes, scale);
  r.w = fp4x2_to_bf16x2<3>(codes, scale);
  return r;
}

// Two floats as a packed bf16 pair (first in the low half), rounded to nearest even
// by the hardware convert (the same bits as f32_to_bf16_rne for every non-NaN input).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  const bf2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// bf16 head and residual of two weights (hardware round-to-nearest-even), packed with
// the first weight in the low half: head + residual carries 16 significant bits.
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  const bf2 h = {(__bf16)p0, (__bf16)p1};
  hi = __builtin_bit_cast(uint32_t, h);
  const float r0 = p0 - __uint_as_float(hi << 16), r1 = p1 - __uint_as_float(hi & 0xffff0000u);
  const bf2 l = {(__bf16)r0, (__bf16)r1};
  lo = __builtin_bit_cast(uint32_t, l);
}

// Order-preserving map of an fp32 score onto uint32 (larger score -> larger key).
// -0 is folded onto +0 so that equal scores give equal keys.  Key 0 is reserved for
// "no entry" (it would be a NaN pattern).
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t b = __float_as_uint(s + 0.0f);   // -0 + 0 = +0 under round-to-nearest
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);   // negative: ~b, else b | sign
}

// max(x, 0) for a non-NaN float, as one integer max on its bits: every negative
// float (and -0) has a negative int32 pattern and maps to +0.
__device__ __forceinline__ float relu0(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

// Wave-wide reductions over 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Unsigned min / max over the 64 lanes of a wave with DPP (pairs, quads, half rows,
// rows, then the row broadcasts); the result is read from lane 63 and returned
// wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));    // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));    // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));   // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));   // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  const int id = -1;   // 0xffffffff: lanes a row mask leaves out keep it
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0xb1, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x4e, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x141, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x140, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts within rows
// of 16 lanes, then broadcasts of lanes 15 and 31 into the following rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

// Page lookup with bounds checks: returns -1 for an absent or out-of-range page.
__device__ __forceinline__ int page_of(const int32_t* __restrict__ block_table, int max_pages,
                                       int n_pages, int b, int entry) {
  int pi = entry >> 6;
  if (entry < 0 || pi >= max_pages) return -1;
  int p = block_table[(int64_t)b * max_pages + pi];
  return (p >= 0 && p < n_pages) ? p : -1;
}

}  // namespace csa2
