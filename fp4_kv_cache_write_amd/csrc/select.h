// Exact workgroup-level top-K over uint32 keys held in registers.
//
// Keys are order-preserving images of fp32 scores (score_key); key 0 marks "no
// entry".  Thread t holds the keys of positions t*KPT .. t*KPT+KPT-1 (blocked
// layout).  The K largest keys are found by an MSB-first radix select over the
// offsets of the keys from the smallest valid key, in digits of up to 11 bits.
// The select yields a threshold key T and the number k_eq of keys equal to
// T that still belong to the top K.  Selected positions are then emitted in
// ascending order: every key above T, and among keys equal to T the k_eq lowest
// positions -- the "larger score first, lower index on ties" order of the
// indexer top-K and the HSI block ranking ([P1] §2.3.4; the pages leave ties open,
// lower index is this library's rule).
#pragma once

#include "common.h"

namespace csa2 {

// LDS the select needs: two histogram buffers + scratch [64 + 8] (per-wave values,
// then the search results and the count of keys tied at the top).  A buffer holds
// 2048 bins with four pad words after every 32 (bin d lives at d + 4*(d/32)): the
// search wave's lane l reads bins 32l..32l+31 as eight aligned 16-byte loads, and
// any 8 consecutive lanes of such a load cover the 32 banks once.
constexpr int kHistStride = 2048 + 4 * 64;
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

// Radix select with two histogram buffers.  Digits are taken from v = key - kmin,
// where [kmin, kmax] is the range of the valid keys (v orders like the key): the
// first digit spans the top 11 bits of that range, so candidates crowded into a
// narrow score range (the chunk winners a merge selects from) still spread over all
// bins instead of piling their LDS atomics onto a handful of counters.  Later digits
// take the next 11 bits until none are left.  Every pass is "all threads add their
// keys, barrier, wave 0 finds the bin holding the K-th key while the other waves
// clear the next pass's buffer, barrier".  The histogram always has 2048 bins and
// the search reads all of them unconditionally (a digit narrower than 11 bits only
// leaves high bins empty), so its LDS reads issue back to back.
template <int NT, int KPT>
__device__ SelectResult block_select(const uint32_t (&key)[KPT], int K, uint32_t* hist, uint32_t* scratch) {
  static_assert(NT >= 128, "needs a second wave to clear buffers");
  static_assert(NT / 64 <= 32, "range scratch holds one min and one max per wave");
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t* res = scratch + 64;
  uint32_t kl = 0xffffffffu, kh = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const uint32_t x = key[i];
    kl = x != 0u ? min(kl, x) : kl;
    kh = max(kh, x);
  }
  kl = wave_min_u32(kl);
  kh = wave_max_u32(kh);
  if (lane == 0) {
    scratch[wid] = kl;
    scratch[32 + wid] = kh;
  }
  if (tid == 0) res[4] = 0u;                                      // keys equal to the largest key
  for (int i = tid; i < kSelectHist; i += NT) hist[i] = 0u;
  __syncthreads();
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    kmin = min(kmin, scratch[w]);
    kmax = max(kmax, scratch[32 + w]);
  }
  if (kmax == 0u) return SelectResult{0u, 0u, 0u};                // no valid key
  const uint32_t range = kmax - kmin;
  int left = range == 0u ? 0 : 32 - __builtin_clz(range);         // bits of v still to resolve
  uint32_t prefix = 0u, mask = 0u, k = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int width = min(left, 11);
    const int shift = left - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* H = hist + (pass & 1) * kHistStride;
    // Many keys tied at the largest key (a sequence whose indexer weights are all
    // negative scores every entry <= 0, and the entries whose head dots are all <= 0
    // tie at exactly 0) put one digit on most lanes, and 64 same-address LDS atomics
    // in one instruction serialise.  A wave whose first key slot has 16 or more lanes
    // on the largest key's digit counts that digit with one atomic per slot; every
    // other key (and every key of other waves) is added on its own.
    const uint32_t vmax = kmax - kmin;
    const bool top_in = (vmax & mask) == prefix;
    const uint32_t hotd = (vmax >> shift) & dmask;
    bool agg;
    {
      const uint32_t x = key[0];
      const bool in = x != 0u && ((x - kmin) & mask) == prefix;
      agg = top_in && __popcll(__ballot(in && (((x - kmin) >> shift) & dmask) == hotd)) >= 16;
    }
    if (pass == 0) {
      // keys equal to kmax: if there are K of them, they alone are the top K
      uint32_t ctop = 0;
#pragma unroll
      for (int i = 0; i < KPT; ++i) ctop += (uint32_t)__popcll(__ballot(key[i] == kmax));
      if (lane == 0 && ctop != 0u) atomicAdd(&res[4], ctop);
    }
    if (agg) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t x = key[i];
        const uint32_t v = x - kmin;
        const bool in = x != 0u && (v & mask) == prefix;
        const uint32_t d = (v >> shift) & dmask;
        const uint64_t same = __ballot(in && d == hotd);
        if (in && d != hotd) atomicAdd(&H[d + 4 * (d >> 5)], 1u);
        if (same != 0ull && lane == __builtin_ctzll(same)) atomicAdd(&H[hotd + 4 * (hotd >> 5)], (uint32_t)__popcll(same));
      }
    } else {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const uint32_t x = key[i];
        const uint32_t v = x - kmin;
        if (x != 0u && (v & mask) == prefix) {
          const uint32_t d = (v >> shift) & dmask;
          atomicAdd(&H[d + 4 * (d >> 5)], 1u);
        }
      }
    }
    __syncthreads();
    if (tid < 64) {
      // Two-level search.  Lane l owns bins [32l, 32l+32): one prefix scan over the
      // lane sums finds the lane holding the K-th key, a second one over that lane's
      // bins (one bin per lane) finds the bin.  "above" = keys in higher bins.
      const u32x4* hl = reinterpret_cast<const u32x4*>(H + lane * 36);
      uint32_t ls = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x4 v = hl[j];
        ls += v.x + v.y + v.z + v.w;
      }
      const uint32_t pre = wave_incl_scan(ls);
      const uint32_t tot = __builtin_amdgcn_readlane(pre, 63);
      const uint32_t above_l = tot - pre;                       // keys in lanes above l
      const uint64_t hit = __ballot(above_l < k && k <= above_l + ls);
      const int ls_lane = __builtin_ctzll(hit);                 // exactly one lane
      const uint32_t above0 = __builtin_amdgcn_readlane(above_l, ls_lane);
      const int bin = ls_lane * 32 + lane;
      const uint32_t cb = lane < 32 ? H[bin + 4 * (bin >> 5)] : 0u;
      const uint32_t pre2 = wave_incl_scan(cb);
      const uint32_t tot2 = __builtin_amdgcn_readlane(pre2, 63);
      const uint32_t above_b = above0 + tot2 - pre2;            // keys in higher bins
      const uint64_t hit2 = __ballot(lane < 32 && above_b < k && k <= above_b + cb);
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
    if (pass == 0 && res[4] >= (uint32_t)K) return SelectResult{kmax, (uint32_t)K, (uint32_t)K};   // K tied at the top
    const uint32_t d = res[0], knew = res[1], in_bin = res[2];
    const uint32_t lo = prefix | (d << shift);                  // smallest v of the bin
    if (knew == in_bin) return SelectResult{kmin + lo - 1u, 0u, (uint32_t)K};   // the whole bin is in
    if (shift == 0) return SelectResult{kmin + lo, knew, (uint32_t)K};          // equal keys, split by position
    prefix = lo;
    mask |= dmask << shift;
    k = knew;
    left = shift;
  }
  return SelectResult{kmin + prefix, k, (uint32_t)K};   // not reached: 3 passes resolve 32 bits
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
