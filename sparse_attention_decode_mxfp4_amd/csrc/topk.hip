// Exact top-k block selection per query row.
//
// ATOM PR #2686 ("Enable Mono decode with fixed DSpark verify", the review
// thread's commit message: each sparse layer selects its own sparse blocks)
// and PR #2812 (a selected block is one page-128 page in the sparse table).
// The k highest scores win; equal scores go to the lower block id; a row with
// no more than k candidates keeps all of them; ids are written ascending,
// padded with -1.
//
// One wave per row. Keys are the scores mapped to order-preserving uint32
// (NaN ranks lowest), all loaded into registers up front. Candidate i lives in
// lane i % 64, so each lane holds every 64th candidate and its maximum bounds
// its group:
//   1. the k-th largest of the 64 lane maxima, T0, is a lower bound of the
//      k-th largest score (k lanes each hold a score >= T0);
//   2. every candidate with key >= T0 is compacted into LDS in index order
//      (ballot + prefix count); typically a few dozen survive;
//   3. each survivor's rank by (key descending, index ascending) is counted
//      against all survivors (in registers, one survivor per lane, when at
//      most 64 survive; through LDS otherwise); rank < k is selected, and since
//      the survivors are in index order a prefix count of the selected ones
//      places each id.
#include "common.hpp"
#include "launch.hpp"

namespace mxs {

__device__ __forceinline__ uint32_t order_key(float f) {        // branch-free
  const uint32_t u = f2u(f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? 1u : k;          // NaN: below every number
}

__device__ __forceinline__ uint32_t wave_prefix_count(bool pred) {   // lanes below me with pred
  const uint64_t m = __ballot(pred);
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int ITEMS>   // candidates per lane: n_cand <= 64 * ITEMS
__global__ __launch_bounds__(64) void k_topk(const float *__restrict__ scores,
                                             const int32_t *__restrict__ context_lens, int32_t stride,
                                             int32_t q, int32_t topk, int32_t *__restrict__ block_table) {
  __shared__ uint32_t s_key[64 * ITEMS];
  __shared__ uint16_t s_idx[64 * ITEMS];
  const int row = blockIdx.x;
  const int b = row / q, j = row % q;
  const int lane = threadIdx.x;
  const int pos = context_lens[b] - q + j;
  int n_cand = pos < 0 ? 0 : pos / kTokens + 1;
  if (n_cand > stride) n_cand = stride;
  const float *s = scores + (int64_t)row * stride;
  int32_t *out = block_table + (int64_t)row * topk;

  if (n_cand <= topk) {
    for (int i = lane; i < topk; i += 64) out[i] = i < n_cand ? i : -1;
    return;
  }
  // all loads in flight at once: candidate lane + 64 r sits in key[r]
  uint32_t key[ITEMS];
  {
    float v[ITEMS];
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) v[r] = s[min(lane + 64 * r, n_cand - 1)];   // clamped, unconditional
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) asm volatile("" : "+v"(v[r]));   // keep every load ahead of the guards
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) key[r] = lane + 64 * r < n_cand ? order_key(v[r]) : 0u;
  }
  // 1. lane maxima and their k-th largest (bitonic sort of 64 values, descending)
  uint32_t v = 0u;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) v = max(v, key[r]);
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int st = size >> 1; st > 0; st >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)v, st);
      const bool lower = (lane & st) == 0;
      const bool desc_block = (lane & size) == 0;
      v = (lower == desc_block) ? max(v, o) : min(v, o);
    }
  }
  const uint32_t T0 = (uint32_t)__shfl((int)v, topk - 1);

  // 2. compact the survivors (key >= T0) in index order
  uint32_t n_surv = 0;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int i = lane + 64 * r;
    const bool keep = i < n_cand && key[r] >= T0;
    const uint32_t at = n_surv + wave_prefix_count(keep);
    if (keep) {
      s_key[at] = key[r];
      s_idx[at] = (uint16_t)i;
    }
    n_surv += (uint32_t)__popcll(__ballot(keep));
  }
  __syncthreads();

  // 3. rank every survivor by (key descending, index ascending); rank < k is
  //    selected, and since survivors are in index order a prefix count of the
  //    selected ones places each id.
  if (n_surv <= 64) {                            // usual case: one survivor per lane, ranks in registers
    const bool have = (uint32_t)lane < n_surv;
    const uint32_t kme = have ? s_key[lane] : 0u;
    const uint32_t ime = have ? s_idx[lane] : 0u;
    uint32_t rank = 0;
#pragma unroll 8
    for (uint32_t o = 0; o < n_surv; ++o) {
      const uint32_t ko = (uint32_t)__builtin_amdgcn_readlane((int)kme, (int)o);
      rank += (ko > kme) || (ko == kme && o < (uint32_t)lane);
    }
    const bool sel = have && rank < (uint32_t)topk;
    const uint32_t at = wave_prefix_count(sel);
    if (sel) out[at] = (int32_t)ime;
    return;
  }
  uint32_t n_out = 0;                            // many ties at the bound: rank through LDS
  for (uint32_t base = 0; base < n_surv; base += 64) {
    const uint32_t me = base + lane;
    bool sel = false;
    if (me < n_surv) {
      const uint32_t kme = s_key[me];
      uint32_t rank = 0;
      for (uint32_t o = 0; o < n_surv && rank < (uint32_t)topk; ++o) {
        const uint32_t ko = s_key[o];
        rank += (ko > kme) || (ko == kme && o < me);
      }
      sel = rank < (uint32_t)topk;
    }
    const uint32_t at = n_out + wave_prefix_count(sel);
    if (sel) out[at] = s_idx[me];
    n_out += (uint32_t)__popcll(__ballot(sel));
  }
}

hipError_t launch_topk(const CacheView &c, const float *scores, int32_t B, int32_t q, int32_t topk,
                       int32_t *block_table, hipStream_t s) {
  if (B * q == 0) return hipSuccess;
  const dim3 grid((unsigned)(B * q));
  if (c.stride <= 64 * 8)
    hipLaunchKernelGGL(k_topk<8>, grid, dim3(64), 0, s, scores, c.context_lens, c.stride, q, topk, block_table);
  else if (c.stride <= 64 * 32)
    hipLaunchKernelGGL(k_topk<32>, grid, dim3(64), 0, s, scores, c.context_lens, c.stride, q, topk, block_table);
  else
    hipLaunchKernelGGL(k_topk<128>, grid, dim3(64), 0, s, scores, c.context_lens, c.stride, q, topk, block_table);
  return hipGetLastError();
}

}  // namespace mxs
