// Exact workgroup-level top-K over uint32 keys held in LDS.
//
// Keys are order-preserving images of fp32 scores (score_key); key 0 marks "no
// entry".  The K largest keys are found by an MSB-first radix select (8-bit
// digits, histogram in LDS replicated R ways to spread atomics), which yields a
// threshold key T and the number k_eq of keys equal to T that still belong to the
// top K.  Selected items are then emitted in ascending position order: every key
// above T, and among keys equal to T the k_eq with the lowest positions -- the
// "larger score first, lower index on ties" order of the indexer top-K and the HSI
// block ranking ([P1] §2.3.4, ties unspecified there; lower index is this
// library's rule).
#pragma once

#include "common.h"

namespace csa2 {

struct SelectSmem {
  uint32_t* hist;   // [256 * R]
  uint32_t* misc;   // [512]: bin totals, results, per-wave round counts
};

// Result: selected entries satisfy key > thr, or key == thr and rank among equal
// keys (in position order) < krem.  `count` is the number selected (min(K, #valid)).
struct SelectResult {
  uint32_t thr;
  uint32_t krem;
  uint32_t count;
};

template <int NT>
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  v = wave_sum_u32(v);
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wid] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += scratch[i];
  __syncthreads();
  return t;
}

template <int NT, int R>
__device__ SelectResult block_select(const uint32_t* __restrict__ keys, int N, int K, SelectSmem sm) {
  static_assert((R & (R - 1)) == 0 && R <= 64, "replicas");
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t k = (uint32_t)K;
  uint32_t* tot = sm.misc;           // [256]
  uint32_t* res = sm.misc + 256;     // [4]
  uint32_t valid = 0;
  SelectResult out{0u, 0u, 0u};
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256 * R; i += NT) sm.hist[i] = 0u;
    __syncthreads();
    const uint32_t rep = (uint32_t)(tid & (R - 1));
    for (int v = tid; v < N; v += NT) {
      const uint32_t key = keys[v];
      if (key != 0u && (key & mask) == prefix)
        atomicAdd(&sm.hist[((key >> shift) & 255u) * R + rep], 1u);
    }
    __syncthreads();
    for (int bin = tid; bin < 256; bin += NT) {
      uint32_t s = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) s += sm.hist[bin * R + r];
      tot[bin] = s;
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 4l..4l+3; "above" = keys in higher bins of this prefix
      const int l = tid;
      const uint32_t c0 = tot[4 * l], c1 = tot[4 * l + 1], c2 = tot[4 * l + 2], c3 = tot[4 * l + 3];
      const uint32_t sl = c0 + c1 + c2 + c3;
      uint32_t suf = sl;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o, kWave);
        if (l + o < 64) suf += t;
      }
      const uint32_t excl = suf - sl;
      if (shift == 24 && l == 0) res[2] = suf;   // all valid keys
      const uint32_t above[4] = {excl + c3 + c2 + c1, excl + c3 + c2, excl + c3, excl};
      const uint32_t cnt[4] = {c0, c1, c2, c3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above[i] < k && k <= above[i] + cnt[i]) {
          res[0] = (uint32_t)(4 * l + i);
          res[1] = k - above[i];
          res[3] = cnt[i];
        }
      }
    }
    __syncthreads();
    if (shift == 24) {
      valid = res[2];
      if (valid <= (uint32_t)K) {            // fewer valid keys than K: take them all
        out = SelectResult{0u, 0u, valid};
        __syncthreads();
        return out;
      }
    }
    const uint32_t d = res[0];
    const uint32_t knew = res[1];
    const uint32_t in_bin = res[3];
    __syncthreads();
    const uint32_t lo = prefix | (d << shift);
    if (knew == in_bin) {                    // the whole bin is taken: threshold below it
      out = SelectResult{lo == 0u ? 0u : lo - 1u, 0u, (uint32_t)K};
      return out;
    }
    prefix = lo;
    mask |= 255u << shift;
    k = knew;
  }
  out = SelectResult{prefix, k, (uint32_t)K};
  return out;
}

// Emit selected positions in ascending order: emit(v, pos) for the pos-th selected v.
template <int NT, class Emit>
__device__ void block_emit_ordered(const uint32_t* __restrict__ keys, int N, SelectResult sr,
                                   uint32_t* wave_counts /*[2][2][NT/64]*/, Emit emit) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t out_run = 0, eq_run = 0;
  int parity = 0;
  for (int base = 0; base < N; base += NT, parity ^= 1) {
    const int v = base + tid;
    const uint32_t key = v < N ? keys[v] : 0u;
    const bool gt = key != 0u && key > sr.thr;
    const bool eq = key != 0u && key == sr.thr && sr.krem > 0u;
    const uint64_t mg = __ballot(gt);
    const uint64_t me = __ballot(eq);
    uint32_t* wc = wave_counts + parity * 2 * NW;
    if (lane == 0) {
      wc[wid] = (uint32_t)__popcll(mg);
      wc[NW + wid] = (uint32_t)__popcll(me);
    }
    __syncthreads();
    uint32_t gt_before = (uint32_t)__popcll(mg & lt_mask);
    uint32_t eq_before = (uint32_t)__popcll(me & lt_mask);
    uint32_t gt_tot = 0, eq_tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t g = wc[i], e = wc[NW + i];
      if (i < wid) {
        gt_before += g;
        eq_before += e;
      }
      gt_tot += g;
      eq_tot += e;
    }
    const uint32_t eq_left = sr.krem > eq_run ? sr.krem - eq_run : 0u;
    const bool sel = gt || (eq && eq_before < eq_left);
    if (sel) emit(v, out_run + gt_before + min(eq_before, eq_left));
    out_run += gt_tot + min(eq_tot, eq_left);
    eq_run += eq_tot;
  }
  __syncthreads();
}

}  // namespace csa2
