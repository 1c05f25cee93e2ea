// Exact top-k block selection of one query row by one workgroup of 4 or 8
// waves (NT = 256 or 512 threads).
//
// ATOM PR #2686 ("Enable Mono decode with fixed DSpark verify", the review
// thread's commit message: each sparse layer selects its own sparse blocks)
// and PR #2812 (each block the selection names is one 128-token page).
// The k highest scores win; equal scores go to the lower block id; a row with
// no more than k candidates keeps all of them; ids come out ascending.
//
// Used by the stand-alone top-k kernel and by the decode step's attention
// kernel, which selects its row's blocks itself before attending to them.
//
// Keys are the scores mapped to order-preserving uint32 (NaN ranks lowest).
// Thread t holds candidates t + NT r. Steps:
//   1. T0 = the k-th largest of the NT thread maxima, a lower bound of the
//      k-th largest score (k threads each hold a score >= T0): every wave
//      sorts its 64 maxima, and each wave merges the sorted lists of all waves
//      itself (bitonic half-cleaners, keeping the top 64 of each pair), so no
//      wave waits for another beyond one barrier;
//   2. every candidate with key >= T0 (typically a few dozen) is compacted
//      into LDS in ascending id order (id = tid + NT r ascends with (r, wave,
//      lane): per-(r, wave) ballot counts, one barrier for the counts);
//   3. exactly k survivors are the selection, already ascending; when at most
//      64 survive, every wave holds them one per lane, finds the k-th largest
//      key T1 (a sort of the keys across the lanes), keeps the keys above T1
//      and, of those equal to T1, the lowest ids (lane order), and packs the
//      kept ids to the front (one forward lane permute), which leaves them
//      ascending; with more survivors (ties at the bound) each survivor is
//      ranked against all of them through LDS and the ids are sorted after.
#pragma once

#include "common.hpp"

namespace mxs {

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

// Workgroup barrier for LDS data only: the LDS writes are waited for, vector
// memory operations are not (unlike __syncthreads, which would also wait for
// every global load still in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int ITEMS, int NW = 4>
struct TopkSmem {
  static constexpr int kThreads = 64 * NW;
  uint32_t key[kThreads * ITEMS];          // survivors, ascending id
  uint16_t idx[kThreads * ITEMS];
  uint32_t wmax[NW][64];                   // each wave's thread maxima, sorted descending
  alignas(16) uint32_t wcnt[ITEMS][NW];    // survivors of item r in wave w (read 16 B at a time)
  uint32_t by_rank[64];                    // many-survivor path: id of rank r
};

// The top 64 of the sorted (descending) lists of waves [W0, W0 + N), sorted
// DESC (or ascending): pairs of lists are merged with a bitonic half-cleaner
// that keeps the larger half.
template <bool DESC, int W0, int N, int NW>
__device__ __forceinline__ uint32_t top64_of_waves(const uint32_t (&wmax)[NW][64], int lane) {
  if constexpr (N == 1) {
    return DESC ? wmax[W0][lane] : wmax[W0][63 - lane];
  } else {
    const uint32_t a = top64_of_waves<true, W0, N / 2, NW>(wmax, lane);        // descending
    const uint32_t b = top64_of_waves<false, W0 + N / 2, N / 2, NW>(wmax, lane);  // ascending
    return merge64<DESC>(max(a, b));
  }
}

// Selects the top-k of one row; every thread of the workgroup calls it.
// Thread t passes the scores of candidates t + NT r in v[r] (any value where
// t + NT r >= n_cand), 0 <= n_cand <= NT ITEMS, 1 <= topk <= 64. Every wave
// gets back, in lane s < n_sel = min(topk, n_cand), the s-th smallest selected
// block id (other lanes: 0xFFFFFFFF, or the lane number when n_cand <= topk).
template <int ITEMS, int NW>
__device__ __forceinline__ uint32_t wg_topk(const float (&v)[ITEMS], int n_cand, int topk, TopkSmem<ITEMS, NW> &sm,
                                            int &n_sel) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (n_cand <= topk) {                      // every candidate is selected
    n_sel = n_cand;
    return (uint32_t)lane;
  }
  n_sel = topk;
  uint32_t key[ITEMS];
  uint32_t m = 0u;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    key[r] = tid + NT * r < n_cand ? order_key(v[r]) : 0u;
    m = max(m, key[r]);
  }
  // 1. T0: the k-th largest of the NT thread maxima
  sm.wmax[wave][lane] = sort64<true>(m);
  lds_barrier();
  const uint32_t e = top64_of_waves<true, 0, NW, NW>(sm.wmax, lane);
  const uint32_t T0 = (uint32_t)__builtin_amdgcn_readlane((int)e, topk - 1);

  // 2. compact the survivors in ascending id order: item r of wave w lands
  //    after every survivor of items < r and of item r in waves < w
  bool keep[ITEMS];
  uint32_t at[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    keep[r] = tid + NT * r < n_cand && key[r] >= T0;
    const uint64_t bal = __ballot(keep[r]);
    at[r] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    if (lane == 0) sm.wcnt[r][wave] = (uint32_t)__popcll(bal);
  }
  lds_barrier();
  uint32_t n_surv = 0;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    uint32_t below = 0, all = 0;
#pragma unroll
    for (int w4 = 0; w4 < NW; w4 += 4) {
      const u32x4 c = *reinterpret_cast<const u32x4 *>(&sm.wcnt[r][w4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        below += wave > w4 + i ? c[i] : 0u;
        all += c[i];
      }
    }
    const uint32_t base = n_surv + below;
    n_surv += all;
    if (keep[r]) {
      sm.key[base + at[r]] = key[r];
      sm.idx[base + at[r]] = (uint16_t)(tid + NT * r);
    }
  }
  lds_barrier();

  // 3. exact selection by (key descending, id ascending), ids kept ascending
  if (n_surv == (uint32_t)topk)              // exactly k survive: all selected
    return (uint32_t)lane < n_surv ? (uint32_t)sm.idx[lane] : 0xFFFFFFFFu;
  if (n_surv <= 64u) {
    const bool have = (uint32_t)lane < n_surv;
    const uint32_t ks = have ? sm.key[lane] : 0u, is = have ? (uint32_t)sm.idx[lane] : 0xFFFFFFFFu;
    const uint32_t T1 = (uint32_t)__builtin_amdgcn_readlane((int)sort64<true>(ks), topk - 1);
    const uint64_t gt = __ballot(have && ks > T1), eq = __ballot(have && ks == T1);
    const uint32_t eq_below =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
    const bool take = have && (ks > T1 || (ks == T1 && eq_below < (uint32_t)topk - (uint32_t)__popcll(gt)));
    // stable partition: taken lanes to the front (ascending ids), the rest after
    const uint64_t tb = __ballot(take);
    const uint32_t before = __builtin_amdgcn_mbcnt_hi((uint32_t)(tb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)tb, 0u));
    const uint32_t dst = take ? before : (uint32_t)__popcll(tb) + (uint32_t)lane - before;
    const uint32_t got = (uint32_t)__builtin_amdgcn_ds_permute((int)(dst * 4u), (int)is);
    return lane < topk ? got : 0xFFFFFFFFu;
  }
  // ties at the bound: rank through LDS, then sort the selected ids
  for (uint32_t i = tid; i < n_surv; i += NT) {
    const uint32_t ki = sm.key[i], ii = sm.idx[i];
    uint32_t rank = 0;
    for (uint32_t o = 0; o < n_surv; ++o) {
      const uint32_t ko = sm.key[o];
      rank += (ko > ki) || (ko == ki && sm.idx[o] < ii);
    }
    if (rank < (uint32_t)topk) sm.by_rank[rank] = ii;
  }
  lds_barrier();
  return sort64<false>(lane < topk ? sm.by_rank[lane] : 0xFFFFFFFFu);   // ascending ids
}

}  // namespace mxs
