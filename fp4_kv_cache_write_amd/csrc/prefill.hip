// Chunked prefill: the causal Full indexer of every chunk query, then the sparse
// gather-attention of every chunk query (the decode attention kernel, run with C
// queries per sequence and window rows read from the caller's `local` array).
//
// [P1] "DeepSeek-v4.1 Flash: KVキャッシュ圧縮の限界を押し広げる" §2.3.1 (each query
// scores every entry its causal mask lets it see and keeps the top K), §2.2 (the
// prefill cost is what the compression targets); [P3] "DeepSeek V4.1 Flash
// architecture..." (causal mask: a query sees only entries whose tokens precede it).
//
// Indexer (prefill_index_kernel): one wave per (sequence, 4 consecutive queries).
// The 4 queries x 4 indexer heads fill the 16 rows of a 16x16x32 bf16 MFMA, so a
// 16-entry key group costs two MFMAs and every lane ends with one finished score:
// lane l holds query l/16 against entry l%16 (rows 4q..4q+3 of the accumulator are
// query q's heads).  Keys stream page by page straight from the paged cache, two
// pages ahead of the MFMAs, as buffer loads off a descriptor of the page (the page
// base in scalar registers, constant lane offsets: no vector ALU work per load);
// page ids come 64 at a time in one vector load and are read out with v_readlane.
//
// Top-K per query is streamed: every query keeps a list of (key, entry) pairs in
// the workspace, in entry order, and a threshold tau.  A score joins the list only
// when it beats tau.  When a list nears capacity the wave loads it into registers,
// selects its K best pairs exactly (MSB-first radix select over 8-bit digits in an
// LDS histogram, ties to the lower entry) and writes them back in entry order; tau
// becomes the smallest kept key.  This is exact: every dropped pair, and every later
// pair that does not beat tau, has K pairs ranked above it (equal keys rank by
// entry, and later pairs have higher entries).  At the end the same select writes
// the K entries in ascending order.  Keeping the lists out of LDS leaves the
// occupancy to the register budget, so enough waves are resident to cover the
// latency of the key stream.
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

// Sets of 4 queries per wave (4 queries x 4 heads fill an MFMA's rows); the keys are
// converted once for all sets.  Measured on the MI355X at 4 x 4,096 queries over
// 131,072 prior tokens, 2 sets run 7% slower than 1: 136 registers leave 3 waves per
// SIMD, and half as many waves hide less of the key stream's latency.
constexpr int kPfSets = 1;
constexpr int kPfQ = 4 * kPfSets;   // queries per wave
constexpr int kPfHist = 256;   // radix-select histogram bins (8-bit digits)

struct PfIndexArgs {
  const uint8_t* idx_codes;
  const uint8_t* idx_scales;
  const int32_t* block_table;
  int n_pages, max_pages;
  const int32_t* prior_len;
  int64_t max_ctx;
  const uint16_t* q_idx;
  const uint16_t* w_idx;
  int C, topk, cap;
  u32x2* lists;          // [B*C][cap] (key, entry) pairs
  int32_t* topk_idx;
  int n_units, per_xcd;
};

template <bool B>
struct Check {
  static constexpr bool value = B;
};

// Number of set bits of m at lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Selected: key > thr, or key == thr among the first krem such keys in list order.
struct WaveSel {
  uint32_t thr, krem;
};

// Exact selection of the k largest nonzero keys of kst[0..cnt) (at least k + 1 of
// them) by one wave.  Lane l owns histogram bins 4l..4l+3, so a scan over the lane
// sums finds the lane holding the k-th key and four compares find the bin.
__device__ WaveSel wave_select(const uint32_t* kst, int cnt, uint32_t k, uint32_t* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0u, mask = 0u;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    for (int p = lane; p < cnt; p += 64) {
      const uint32_t x = kst[p];
      if (x != 0u && (x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    const u32x4 c = *reinterpret_cast<const u32x4*>(hist + 4 * lane);
    const uint32_t ls = c.x + c.y + c.z + c.w;
    const uint32_t incl = wave_incl_scan(ls);
    const uint32_t above_l = __builtin_amdgcn_readlane(incl, 63) - incl;   // keys in higher lanes
    const uint64_t hit = __ballot(above_l < k && k <= above_l + ls);
    const int hl = (int)(__builtin_ctzll(hit | (1ull << 63)));
    const uint32_t cs[4] = {c.x, c.y, c.z, c.w};
    uint32_t above = above_l, bin = 0u, knew = 0u, inb = 0u;
    bool found = false;
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (!found && above < k && k <= above + cs[j]) {
        found = true;
        bin = 4u * lane + j;
        knew = k - above;
        inb = cs[j];
      }
      above += cs[j];
    }
    bin = __builtin_amdgcn_readlane(bin, hl);
    knew = __builtin_amdgcn_readlane(knew, hl);
    inb = __builtin_amdgcn_readlane(inb, hl);
    const uint32_t lo = prefix | (bin << shift);
    __syncthreads();
    if (knew == inb) return WaveSel{lo ? lo - 1u : 0u, 0u};   // the whole bin is in
    prefix = lo;
    mask |= 255u << shift;
    k = knew;
  }
  return WaveSel{prefix, k};
}

// Keep the selected pairs of list[0..cnt) in order -- back into the list (out ==
// nullptr) or as entry ids into out -- and return how many were kept; *kmin gets
// the smallest kept key.  sel_all keeps every pair.  Keys and entry ids are copied
// into the wave's LDS areas kst and kid with direct global->LDS loads, all issued
// before the one wait, so a compaction costs one memory round trip.
__device__ int list_keep(u32x2* list, int cnt, int topk, bool sel_all, uint32_t* kst, uint32_t* kid,
                         uint32_t* hist, int32_t* out, uint32_t* kmin) {
  const int lane = threadIdx.x & 63;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(list);
  const int nr = (cnt + 63) >> 6;
  for (int r = 0; r < nr; ++r) {
    const int p = 64 * r + lane;
    if (p < cnt) {
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(words + 2 * p), kst + 64 * r, 4, 0, 0);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(words + 2 * p + 1), kid + 64 * r, 4, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const WaveSel s = sel_all ? WaveSel{0u, 0u} : wave_select(kst, cnt, (uint32_t)topk, hist);
  uint32_t kept = 0u, eq_before = 0u, mn = 0xffffffffu;
#pragma unroll 1
  for (int r = 0; r < nr; ++r) {
    const int p = 64 * r + lane;
    const uint32_t x = p < cnt ? kst[p] : 0u;
    const bool eq = x != 0u && x == s.thr;
    const uint64_t meq = __ballot(eq);
    const bool sel = x != 0u && (x > s.thr || (eq && eq_before + lanes_below(meq) < s.krem));
    const uint64_t ms = __ballot(sel);
    const uint32_t dst = kept + lanes_below(ms);
    const int32_t id = sel ? (int32_t)kid[p] : -1;
    if (sel) {
      if (out) {
        out[dst] = id;
      } else {
        list[dst] = u32x2{x, (uint32_t)id};
      }
      mn = min(mn, x);
    }
    kept += (uint32_t)__builtin_popcountll(ms);
    eq_before += (uint32_t)__builtin_popcountll(meq);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
  __syncthreads();   // kst is reused by the next call
  *kmin = mn;
  return (int)kept;
}

__global__ __launch_bounds__(64) void prefill_index_kernel(PfIndexArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t pf_lds[];
  uint32_t* hist = pf_lds;             // [256]
  uint32_t* kst = pf_lds + kPfHist;    // [cap] keys of the list being compacted
  uint32_t* kid = kst + a.cap;         // [cap] its entry ids
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int unit = xcd * a.per_xcd + slot;   // contiguous query groups per XCD
  if (slot >= a.per_xcd || unit >= a.n_units) return;
  const int qpb = (a.C + kPfQ - 1) / kPfQ;
  const int b = unit / qpb;
  const int i0 = (unit - b * qpb) * kPfQ;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;

  int64_t prior = a.prior_len[b];
  if (prior < 0) prior = 0;
  auto n_vis = [&](int i) -> int {   // entries visible to chunk query i
    if (i >= a.C) return 0;
    int64_t L = prior + i + 1;
    if (L > a.max_ctx) L = a.max_ctx;
    return (int)(L >> 1);
  };
  // Query set s (s < kPfSets) is queries i0 + 4s .. i0 + 4s + 3; lane l's query in set
  // s is i0 + 4s + l/16.
  int nv[kPfSets];
#pragma unroll
  for (int st = 0; st < kPfSets; ++st) nv[st] = n_vis(i0 + 4 * st + g);
  // fewest entries seen by any query of the wave (0 when the chunk ends inside the group)
  const int nv_min = (i0 + kPfQ - 1 < a.C) ? n_vis(i0) : 0;
  const int nv_max = n_vis(min(i0 + kPfQ - 1, a.C - 1));

  // A operands of set s: row m = l%16 is head m%4 of query i0 + 4s + m/4, dims 16g .. 16g+15.
  bf16x8 qa[kPfSets][2];
  float wh[kPfSets][4];
#pragma unroll
  for (int st = 0; st < kPfSets; ++st) {
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    const int qr = i0 + 4 * st + (n >> 2);
    if (qr < a.C) {
      const uint16_t* qp = a.q_idx + (((int64_t)b * a.C + qr) * CSA2_H_INDEX + (n & 3)) * CSA2_D_INDEX + 16 * g;
      v0 = *reinterpret_cast<const u32x4*>(qp);
      v1 = *reinterpret_cast<const u32x4*>(qp + 8);
    }
    qa[st][0] = __builtin_bit_cast(bf16x8, v0);
    qa[st][1] = __builtin_bit_cast(bf16x8, v1);
#pragma unroll
    for (int h = 0; h < 4; ++h) wh[st][h] = 0.f;
    if (i0 + 4 * st + g < a.C) {
#pragma unroll
      for (int h = 0; h < 4; ++h)
        wh[st][h] = bf16_to_f32(a.w_idx[((int64_t)b * a.C + i0 + 4 * st + g) * CSA2_H_INDEX + h]);
    }
  }

  // the lane's list in each set, its threshold (as a key and as a score) and fill
  u32x2* const list0 = a.lists + ((int64_t)b * a.C + i0) * a.cap;
  float tau_s[kPfSets];   // a score beats tau iff it exceeds tau_s
  int cnt[kPfSets];
#pragma unroll
  for (int st = 0; st < kPfSets; ++st) {
    tau_s[st] = -INFINITY;
    cnt[st] = 0;
  }

  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int np = (nv_max + CSA2_PAGE - 1) / CSA2_PAGE;
  auto bt_batch = [&](int k) -> int {   // page ids 64k .. 64k+63, one per lane
    const int pi = 64 * k + lane;
    return (pi < np && pi < a.max_pages) ? bt[pi] : -1;
  };
  int bt_cur = bt_batch(0), bt_nxt = bt_batch(1);

  // A page's loads are buffer loads off a descriptor of that page (a page that is
  // absent or out of range reads page 0 and is dropped): the page base sits in scalar
  // registers and every lane's offsets are constants.
  const int voff_code = n * CSA2_IDX_CODE_BYTES + 8 * g;
  const int voff_scale = n * CSA2_IDX_SCALE_BYTES + (g >> 1);
  struct Page {
    u32x2 cd[4];
    uint32_t sb[4];
    int ok;
  };
  auto load_page = [&](int p, int phys, Page& pg) {
    pg.ok = (p < np && phys >= 0 && phys < a.n_pages) ? 1 : 0;
    const int64_t pc = pg.ok ? phys : 0;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.idx_codes + pc * (CSA2_PAGE * CSA2_IDX_CODE_BYTES)), 0,
        CSA2_PAGE * CSA2_IDX_CODE_BYTES, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.idx_scales + pc * (CSA2_PAGE * CSA2_IDX_SCALE_BYTES)), 0,
        CSA2_PAGE * CSA2_IDX_SCALE_BYTES, 0x00020000);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      pg.cd[t] = __builtin_amdgcn_raw_buffer_load_b64(rc, voff_code + t * 16 * CSA2_IDX_CODE_BYTES, 0, 0);
      pg.sb[t] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff_scale + t * 16 * CSA2_IDX_SCALE_BYTES, 0, 0);
    }
  };
  // Scores the 64 entries of a staged page for the wave's queries (one conversion of
  // the keys serves every set) and appends those above a query's threshold to its
  // list.  Check<true> also tests each entry against the query's visible count.
  auto score_page = [&](const Page& pg, int p, auto chk) {
    // all of the page's products first, then the scores: the MFMAs of the later groups
    // cover the latency of the earlier ones' results
    f32x4 dd[4][kPfSets];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float sc = e8m0_scale(pg.sb[t]);
      u32x4 lo, hi;
      lo.x = fp4x2_to_bf16x2<0>(pg.cd[t].x, sc);
      lo.y = fp4x2_to_bf16x2<1>(pg.cd[t].x, sc);
      lo.z = fp4x2_to_bf16x2<2>(pg.cd[t].x, sc);
      lo.w = fp4x2_to_bf16x2<3>(pg.cd[t].x, sc);
      hi.x = fp4x2_to_bf16x2<0>(pg.cd[t].y, sc);
      hi.y = fp4x2_to_bf16x2<1>(pg.cd[t].y, sc);
      hi.z = fp4x2_to_bf16x2<2>(pg.cd[t].y, sc);
      hi.w = fp4x2_to_bf16x2<3>(pg.cd[t].y, sc);
#pragma unroll
      for (int st = 0; st < kPfSets; ++st) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st][0], __builtin_bit_cast(bf16x8, lo), d, 0, 0, 0);
        dd[t][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st][1], __builtin_bit_cast(bf16x8, hi), d, 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int e = p * CSA2_PAGE + 16 * t + n;
#pragma unroll
      for (int st = 0; st < kPfSets; ++st) {
        const f32x4 d = dd[t][st];
        // lane l: d[i] = head i of query i0 + 4st + l/16 against entry l%16 of the group
        const float s = wh[st][0] * relu0(d[0]) + wh[st][1] * relu0(d[1]) + wh[st][2] * relu0(d[2]) +
                        wh[st][3] * relu0(d[3]);
        const bool app = pg.ok && (!decltype(chk)::value || e < nv[st]) && s > tau_s[st];
        const uint64_t m = __builtin_amdgcn_ballot_w64(app);
        if (m) {
          const uint32_t mg = (uint32_t)(m >> (16 * g)) & 0xffffu;
          u32x2* lq = list0 + (int64_t)(4 * st + g) * a.cap;
          if (app) lq[cnt[st] + __builtin_popcount(mg & ((1u << n) - 1u))] = u32x2{score_key(s), (uint32_t)e};
          cnt[st] += __builtin_popcount(mg);
        }
      }
    }
  };
  Page p0, p1;
  load_page(0, __builtin_amdgcn_readlane(bt_cur, 0), p0);
  load_page(1, __builtin_amdgcn_readlane(bt_cur, 1), p1);

#pragma unroll 1
  for (int p = 0; p < np; ++p) {
    // issue the loads of page p + 2 before scoring page p
    const int lp = p + 2;
    if ((lp & 63) == 0) {
      bt_cur = bt_nxt;
      bt_nxt = bt_batch((lp >> 6) + 1);
    }
    Page p2;
    load_page(lp, __builtin_amdgcn_readlane(bt_cur, lp & 63), p2);

    // only the last pages hold entries that some of the queries cannot see
    if ((p + 1) * CSA2_PAGE <= nv_min) {
      score_page(p0, p, Check<false>{});
    } else {
      score_page(p0, p, Check<true>{});
    }
    p0 = p1;
    p1 = p2;

    // a page adds at most 64 pairs per query: compact before a list could overflow
    bool full = false;
#pragma unroll
    for (int st = 0; st < kPfSets; ++st) full = full || cnt[st] > a.cap - CSA2_PAGE;
    if (__ballot(full)) {
      __threadfence_block();   // the wave's list stores are visible to all its lanes
#pragma unroll
      for (int st = 0; st < kPfSets; ++st) {
#pragma unroll 1
        for (int qq = 0; qq < 4; ++qq) {
          const int c = __builtin_amdgcn_readlane(cnt[st], 16 * qq);
          if (c <= a.cap - CSA2_PAGE) continue;
          uint32_t mn;
          const int kept =
              list_keep(list0 + (int64_t)(4 * st + qq) * a.cap, c, a.topk, false, kst, kid, hist, nullptr, &mn);
          if (g == qq) {
            cnt[st] = kept;
            tau_s[st] = key_score(mn);
          }
        }
      }
      __threadfence_block();
    }
  }

  // final exact top-K of each query, entries ascending, padded with -1
  __threadfence_block();
#pragma unroll
  for (int st = 0; st < kPfSets; ++st) {
#pragma unroll 1
    for (int qq = 0; qq < 4; ++qq) {
      const int qi = 4 * st + qq;
      if (i0 + qi >= a.C) break;
      const int c = __builtin_amdgcn_readlane(cnt[st], 16 * qq);
      int32_t* out = a.topk_idx + ((int64_t)b * a.C + i0 + qi) * a.topk;
      uint32_t mn;
      const int kept = list_keep(list0 + (int64_t)qi * a.cap, c, a.topk, c <= a.topk, kst, kid, hist, out, &mn);
      for (int r = kept + lane; r < a.topk; r += 64) out[r] = -1;
    }
  }
}

// List capacity: K kept pairs plus at least 512 slots of slack.
int pf_cap(int topk) { return (max(topk + 512, 1024) + 63) & ~63; }

}  // namespace

// Workspace: the candidate lists of all chunk queries, then their top-K lists
// (used when the caller passes no topk_idx).
static size_t pf_lists_bytes(int B, int C, int topk) {
  return (((size_t)B * C * pf_cap(topk) * 8) + 255) & ~(size_t)255;
}

size_t prefill_ws(int B, int H, int64_t max_ctx, int topk, int C) {
  (void)H;
  (void)max_ctx;
  return pf_lists_bytes(B, C, topk) + ((((size_t)B * C * topk * 4) + 255) & ~(size_t)255);
}

int launch_prefill_chunk(const csa2_cache_t& c, int B, int H, const int32_t* prior_len,
                         int64_t max_ctx, int C, const uint16_t* q, const uint16_t* q_idx,
                         const uint16_t* w_idx, const uint16_t* local, int W, int topk,
                         float sm_scale, uint16_t* out, int32_t* topk_idx, void* ws, hipStream_t s) {
  u32x2* lists = reinterpret_cast<u32x2*>(ws);
  int32_t* tk = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(ws) +
                                                                  pf_lists_bytes(B, C, topk));
  PfIndexArgs a;
  a.idx_codes = c.idx_codes;
  a.idx_scales = c.idx_scales;
  a.block_table = c.block_table;
  a.n_pages = c.n_pages;
  a.max_pages = c.max_pages;
  a.prior_len = prior_len;
  a.max_ctx = max_ctx;
  a.q_idx = q_idx;
  a.w_idx = w_idx;
  a.C = C;
  a.topk = topk;
  a.cap = pf_cap(topk);
  a.lists = lists;
  a.topk_idx = tk;
  const int64_t units = (int64_t)B * ((C + kPfQ - 1) / kPfQ);
  if (units > 0x0fffffff) return CSA2_EUNSUPPORTED;
  a.n_units = (int)units;
  a.per_xcd = (int)((units + 7) / 8);
  const size_t lds = (size_t)(kPfHist + 2 * a.cap) * 4;
  hipLaunchKernelGGL(prefill_index_kernel, dim3(8u * (unsigned)a.per_xcd), dim3(64), lds, s, a);
  const int rc = hip_status();
  if (rc != CSA2_OK) return rc;
  return launch_gather_attention(c, B, C, H, prior_len, true, q, tk, topk, local, W, sm_scale, out,
                                 nullptr, s);
}

}  // namespace csa2
