// Stand-alone top-k: one 256-thread workgroup per query row runs the
// workgroup selection of topk.hpp and writes the row's block table (ids
// ascending, padded with -1).
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"

namespace mxs {

constexpr int kTopkWaves = 4, kTopkThreads = 64 * kTopkWaves;

template <int ITEMS>   // candidates per thread: n_cand <= 256 * ITEMS
__global__ __launch_bounds__(kTopkThreads) void k_topk(const float *__restrict__ scores,
                                                       const int32_t *__restrict__ context_lens, int32_t stride,
                                                       int32_t q, int32_t topk, int32_t *__restrict__ block_table) {
  __shared__ TopkSmem<ITEMS, kTopkWaves> sm;
  const int row = blockIdx.x;
  const int b = row / q, j = row % q;
  const int tid = threadIdx.x;
  const float *s = scores + (int64_t)row * stride;
  // the scores are requested with the context length (clamped to the row, so
  // unconditional); entries past the row's candidates are ignored
  const int pos = context_lens[b] - q + j;
  float v[ITEMS];
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) v[r] = s[min(tid + kTopkThreads * r, stride - 1)];
  const int n_cand = pos < 0 ? 0 : min(pos / kTokens + 1, (int)stride);
  int n_sel;
  const uint32_t sel = wg_topk<ITEMS, kTopkWaves>(v, n_cand, topk, sm, n_sel);
  if (tid < topk) block_table[(int64_t)row * topk + tid] = tid < n_sel ? (int32_t)sel : -1;
}

hipError_t launch_topk(const CacheView &c, const float *scores, int32_t B, int32_t q, int32_t topk,
                       int32_t *block_table, hipStream_t s) {
  if (B * q == 0) return hipSuccess;
  const dim3 grid((unsigned)(B * q)), block(kTopkThreads);
  if (c.stride <= kTopkThreads * 2)
    hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, scores, c.context_lens, c.stride, q, topk, block_table);
  else if (c.stride <= kTopkThreads * 8)
    hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, scores, c.context_lens, c.stride, q, topk, block_table);
  else
    hipLaunchKernelGGL(k_topk<32>, grid, block, 0, s, scores, c.context_lens, c.stride, q, topk, block_table);
  return hipGetLastError();
}

}  // namespace mxs
