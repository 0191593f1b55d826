// Exact workgroup-level top-K over uint32 keys held in registers.
//
// Keys are order-preserving images of fp32 scores (score_key); key 0 marks "no
// entry".  Thread t holds the keys of positions t*KPT .. t*KPT+KPT-1 (blocked
// layout).  The K largest keys are found by an MSB-first radix select with
// 11/11/10-bit digits; the first digit covers the sign, the exponent and two
// mantissa bits, so even a narrow score range spreads over dozens of histogram
// bins.  The select yields a threshold key T and the number k_eq of keys equal to
// T that still belong to the top K.  Selected positions are then emitted in
// ascending order: every key above T, and among keys equal to T the k_eq lowest
// positions -- the "larger score first, lower index on ties" order of the
// indexer top-K and the HSI block ranking ([P1] §2.3.4; the pages leave ties open,
// lower index is this library's rule).
#pragma once

#include "common.h"

namespace csa2 {

// LDS the select needs: two histogram buffers + scratch [64 + 8].  A buffer holds
// 2048 bins with one pad word after every 32 (bin d lives at d + d/32), so the
// search wave -- lane l reading bins 32l..32l+31 -- touches 64 distinct banks.
constexpr int kHistStride = 2048 + 64;
constexpr int kSelectHist = 2 * kHistStride;
constexpr int kSelectScratch = 72;

// Selected: key > thr, or key == thr among the first krem equal keys (position
// order).  count = min(K, #valid).
struct SelectResult {
  uint32_t thr;
  uint32_t krem;
  uint32_t count;
};

// Exclusive scan over the block in thread order; *total gets the block sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* scratch, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(v);
  if (lane == 63) scratch[wid] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t s = scratch[w];
    before += (w < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + inc - v;
}

// Radix select with two histogram buffers: every pass is "all threads add their
// keys, barrier, wave 0 finds the bin holding the K-th key while the other waves
// clear the next pass's buffer, barrier".
template <int NT, int KPT>
__device__ SelectResult block_select(const uint32_t (&key)[KPT], int K, uint32_t* hist, uint32_t* scratch) {
  static_assert(NT >= 128, "needs a second wave to clear buffers");
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t* res = scratch + 64;
  for (int i = tid; i < kSelectHist; i += NT) hist[i] = 0u;
  __syncthreads();
  uint32_t prefix = 0u, mask = 0u, k = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    uint32_t* H = hist + (pass & 1) * kHistStride;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint32_t x = key[i];
      if (x != 0u && (x & mask) == prefix) {
        const uint32_t d = (x >> shift) & (uint32_t)(nb - 1);
        atomicAdd(&H[d + (d >> 5)], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // Two-level search.  Lane l owns bins [l*bpl, (l+1)*bpl): one prefix scan over
      // the lane sums finds the lane holding the K-th key, a second one over that
      // lane's bins (one bin per lane) finds the bin.  "above" = keys in higher bins.
      const int bpl = nb / 64;
      const uint32_t* hl = H + lane * bpl + ((lane * bpl) >> 5);
      uint32_t ls = 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) ls += (j < bpl) ? hl[j] : 0u;
      const uint32_t pre = wave_incl_scan(ls);
      const uint32_t tot = __builtin_amdgcn_readlane(pre, 63);
      const uint32_t above_l = tot - pre;                       // keys in lanes above l
      const uint64_t hit = __ballot(above_l < k && k <= above_l + ls);
      const int ls_lane = __builtin_ctzll(hit);                 // exactly one lane
      const uint32_t above0 = __builtin_amdgcn_readlane(above_l, ls_lane);
      const int bin = ls_lane * bpl + lane;
      const uint32_t cb = lane < bpl ? H[bin + (bin >> 5)] : 0u;
      const uint32_t pre2 = wave_incl_scan(cb);
      const uint32_t tot2 = __builtin_amdgcn_readlane(pre2, 63);
      const uint32_t above_b = above0 + tot2 - pre2;            // keys in higher bins
      const uint64_t hit2 = __ballot(lane < bpl && above_b < k && k <= above_b + cb);
      const int jb = __builtin_ctzll(hit2);
      if (lane == jb) {
        res[0] = (uint32_t)bin;
        res[1] = k - above_b;
        res[2] = cb;
      }
      if (lane == 0) res[3] = tot;                              // all keys of this pass
    } else {
      uint32_t* other = hist + ((pass + 1) & 1) * kHistStride;
      for (int i = tid - 64; i < kHistStride; i += NT - 64) other[i] = 0u;
    }
    __syncthreads();
    if (pass == 0 && res[3] <= (uint32_t)K) return SelectResult{0u, 0u, res[3]};   // take every valid key
    const uint32_t d = res[0], knew = res[1], in_bin = res[2];
    const uint32_t lo = prefix | (d << shift);
    if (knew == in_bin) return SelectResult{lo == 0u ? 0u : lo - 1u, 0u, (uint32_t)K};
    prefix = lo;
    mask |= (uint32_t)(nb - 1) << shift;
    k = knew;
  }
  return SelectResult{prefix, k, (uint32_t)K};
}

// Emit selected positions in ascending order: emit(i, pos) for the key in slot i of
// this thread (position t*KPT+i) when it is the pos-th selected entry.
template <int NT, int KPT, class Emit>
__device__ __forceinline__ void block_emit(const uint32_t (&key)[KPT], SelectResult sr, uint32_t* scratch, Emit emit) {
  uint32_t gt_c = 0, eq_c = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint32_t x = key[i];
    gt_c += (x != 0u && x > sr.thr) ? 1u : 0u;
    eq_c += (x != 0u && x == sr.thr) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<NT>((gt_c << 16) | eq_c, scratch, &tot);
  uint32_t eq_before = ex & 0xffffu;
  uint32_t out = (ex >> 16) + min(eq_before, sr.krem);
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint32_t x = key[i];
    if (x == 0u) continue;
    if (x > sr.thr) {
      emit(i, out++);
    } else if (x == sr.thr) {
      if (eq_before < sr.krem) emit(i, out++);
      ++eq_before;
    }
  }
}

}  // namespace csa2
