// Exact top-k block selection of one query row by one 256-thread workgroup.
//
// ATOM PR #2686 ("Enable Mono decode with fixed DSpark verify", the review
// thread's commit message: each sparse layer selects its own sparse blocks)
// and PR #2812 (a selected block is one page-128 page in the sparse table).
// The k highest scores win; equal scores go to the lower block id; a row with
// no more than k candidates keeps all of them; ids come out ascending.
//
// Used by the stand-alone top-k kernel and by the decode step's attention
// kernel, which selects its row's blocks itself before attending to them.
//
// Keys are the scores mapped to order-preserving uint32 (NaN ranks lowest).
// Thread t holds candidates t + 256 r. Steps:
//   1. T0 = the k-th largest of the 256 thread maxima, a lower bound of the
//      k-th largest score (k threads each hold a score >= T0): every wave
//      sorts its 64 maxima, and each wave merges the four sorted lists itself
//      (bitonic half-cleaners), so no wave waits for another beyond one barrier;
//   2. every candidate with key >= T0 (typically a few dozen) is compacted
//      into LDS (per-wave ballot offsets, one barrier for the wave totals);
//   3. exactly k survivors are the selection; when at most 64 survive, every
//      wave sorts them by (key descending, id ascending) across its lanes and
//      keeps the first k; with more survivors (ties at the bound) each
//      survivor is ranked against all of them through LDS first; the selected
//      ids are sorted ascending across the lanes.
// All cross-lane exchanges are DPP row permutes and gfx950 permlane swaps
// (no LDS round trip per step).
#pragma once

#include "common.hpp"

namespace mxs {

constexpr int kTopkThreads = 256;

__device__ __forceinline__ uint32_t order_key(float f) {        // branch-free
  const uint32_t u = f2u(f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? 1u : k;          // NaN: below every number
}

// Bitonic networks across the 64 lanes, one value per lane, written as
// template recursion so that every step's lane permute is a compile-time
// choice (a runtime loop over the step distance would dispatch each
// permute through branches).
//
// One stage of the network for blocks of SIZE lanes: compare-exchange at
// distances ST, ST / 2, ..., 1; a block sorts in the final order (DESC: lane
// 0 largest) when (lane & SIZE) == 0 and the other way otherwise (for SIZE =
// 64 every block sorts in the final order: a merge).
template <bool DESC, int SIZE, int ST>
__device__ __forceinline__ uint32_t bitonic_stage(uint32_t v, int lane) {
  if constexpr (ST == 0) {
    return v;
  } else {
    const uint32_t o = xor_lane<ST>(v);
    const bool lower = (lane & ST) == 0;
    const bool first = ((lane & SIZE) == 0) == DESC;
    return bitonic_stage<DESC, SIZE, ST / 2>((lower == first) ? max(v, o) : min(v, o), lane);
  }
}

template <bool DESC, int SIZE = 2>
__device__ __forceinline__ uint32_t sort64(uint32_t v) {
  if constexpr (SIZE > 64) {
    return v;
  } else {
    return sort64<DESC, SIZE * 2>(bitonic_stage<DESC, SIZE, SIZE / 2>(v, threadIdx.x & 63));
  }
}

// A bitonic sequence across the 64 lanes -> sorted.
template <bool DESC>
__device__ __forceinline__ uint32_t merge64(uint32_t v) {
  return bitonic_stage<DESC, 64, 32>(v, threadIdx.x & 63);
}

template <int SIZE, int ST>
__device__ __forceinline__ uint64_t bitonic_stage_desc_u64(uint64_t v, int lane) {
  if constexpr (ST == 0) {
    return v;
  } else {
    const uint64_t o = ((uint64_t)xor_lane<ST>((uint32_t)(v >> 32)) << 32) | xor_lane<ST>((uint32_t)v);
    const bool lower = (lane & ST) == 0;
    const bool first = (lane & SIZE) == 0;
    return bitonic_stage_desc_u64<SIZE, ST / 2>((lower == first) ? (v > o ? v : o) : (v < o ? v : o), lane);
  }
}

template <int SIZE = 2>
__device__ __forceinline__ uint64_t sort64_desc_u64(uint64_t v) {
  if constexpr (SIZE > 64) {
    return v;
  } else {
    return sort64_desc_u64<SIZE * 2>(bitonic_stage_desc_u64<SIZE, SIZE / 2>(v, threadIdx.x & 63));
  }
}

// Workgroup barrier for LDS data only: the LDS writes are waited for, vector
// memory operations are not (unlike __syncthreads, which would also wait for
// every global load still in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int ITEMS>
struct TopkSmem {
  uint32_t key[kTopkThreads * ITEMS];      // survivors (any order)
  uint16_t idx[kTopkThreads * ITEMS];
  uint32_t wmax[4][64];                    // each wave's thread maxima, sorted descending
  uint32_t wtot[4];                        // survivors per wave
  uint32_t by_rank[64];                    // many-survivor path: id of rank r
};

// Selects the top-k of one row; every thread of the 256 calls it. Thread t
// passes the scores of candidates t + 256 r in v[r] (any value where
// t + 256 r >= n_cand), 0 <= n_cand <= 256 ITEMS, 1 <= topk <= 64. Every wave
// gets back, in lane s < n_sel = min(topk, n_cand), the s-th smallest selected
// block id (other lanes: 0xFFFFFFFF, or the lane number when n_cand <= topk).
template <int ITEMS>
__device__ __forceinline__ uint32_t wg_topk(const float (&v)[ITEMS], int n_cand, int topk, TopkSmem<ITEMS> &sm,
                                            int &n_sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n_cand <= topk) {                      // every candidate is selected
    n_sel = n_cand;
    return (uint32_t)lane;
  }
  n_sel = topk;
  uint32_t key[ITEMS];
  uint32_t m = 0u;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    key[r] = tid + kTopkThreads * r < n_cand ? order_key(v[r]) : 0u;
    m = max(m, key[r]);
  }
  // 1. T0: the k-th largest of the 256 thread maxima
  sm.wmax[wave][lane] = sort64<true>(m);
  lds_barrier();
  const uint32_t c = merge64<true>(max(sm.wmax[0][lane], sm.wmax[1][63 - lane]));   // top 64 of waves 0, 1
  const uint32_t d = merge64<false>(max(sm.wmax[2][lane], sm.wmax[3][63 - lane]));  // of waves 2, 3, ascending
  const uint32_t e = merge64<true>(max(c, d));                                        // of all four
  const uint32_t T0 = (uint32_t)__builtin_amdgcn_readlane((int)e, topk - 1);

  // 2. compact the survivors: per-wave ballot offsets, then the wave bases
  bool keep[ITEMS];
  uint32_t at[ITEMS];
  uint32_t wave_n = 0;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    keep[r] = tid + kTopkThreads * r < n_cand && key[r] >= T0;
    const uint64_t bal = __ballot(keep[r]);
    at[r] = wave_n + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    wave_n += (uint32_t)__popcll(bal);
  }
  if (lane == 0) sm.wtot[wave] = wave_n;
  lds_barrier();
  uint32_t base = 0, n_surv = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t n = sm.wtot[w];
    base += w < wave ? n : 0u;
    n_surv += n;
  }
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    if (keep[r]) {
      sm.key[base + at[r]] = key[r];
      sm.idx[base + at[r]] = (uint16_t)(tid + kTopkThreads * r);
    }
  }
  lds_barrier();

  // 3. exact selection by (key descending, id ascending)
  uint32_t sel;
  if (n_surv == (uint32_t)topk) {            // exactly k survive: all selected
    sel = (uint32_t)lane < n_surv ? (uint32_t)sm.idx[lane] : 0xFFFFFFFFu;
  } else if (n_surv <= 64u) {
    const bool have = (uint32_t)lane < n_surv;
    const uint32_t ks = have ? sm.key[lane] : 0u, is = have ? (uint32_t)sm.idx[lane] : 0u;
    const uint64_t comp = sort64_desc_u64(have ? (((uint64_t)ks << 32) | (0xFFFFFFFFu - is)) : 0ull);
    sel = lane < topk ? 0xFFFFFFFFu - (uint32_t)comp : 0xFFFFFFFFu;
  } else {                                   // ties at the bound: rank through LDS
    for (uint32_t i = tid; i < n_surv; i += kTopkThreads) {
      const uint32_t ki = sm.key[i], ii = sm.idx[i];
      uint32_t rank = 0;
      for (uint32_t o = 0; o < n_surv; ++o) {
        const uint32_t ko = sm.key[o];
        rank += (ko > ki) || (ko == ki && sm.idx[o] < ii);
      }
      if (rank < (uint32_t)topk) sm.by_rank[rank] = ii;
    }
    lds_barrier();
    sel = lane < topk ? sm.by_rank[lane] : 0xFFFFFFFFu;
  }
  return sort64<false>(sel);                 // ascending ids
}

}  // namespace mxs
