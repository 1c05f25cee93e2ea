// Stand-alone log-sum-exp merge of split partials: one wave per (query row,
// head); the arithmetic is merge_one (merge.hpp). The decode step merges
// inside its attention launch instead.
#include "common.hpp"
#include "launch.hpp"
#include "merge.hpp"

namespace mxs {

__global__ __launch_bounds__(256) void k_lse_merge(const float *__restrict__ sp_m, const float *__restrict__ sp_l,
                                                   const float *__restrict__ sp_o, int32_t n_rows, int32_t P,
                                                   uint16_t *__restrict__ out, float *__restrict__ lse) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n_rows) return;
  merge_one(sp_m, sp_l, sp_o, r, P, threadIdx.x & 63, out, lse);
}

hipError_t launch_lse_merge(const float *sp_m, const float *sp_l, const float *sp_o, int32_t n_rows, int32_t P,
                            uint16_t *out, float *lse, hipStream_t s) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lse_merge, dim3((unsigned)((n_rows + 3) / 4)), dim3(256), 0, s, sp_m, sp_l, sp_o, n_rows, P,
                     out, lse);
  return hipGetLastError();
}

}  // namespace mxs
