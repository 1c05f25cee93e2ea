// Row store and q store as stand-alone launches (the decode step does both
// inside its scorer launch).
//
// ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches": the
// MXFP4 index-cache commit writes each index-key row into an 8704 B page
// (e8m0 group scale, e2m1 elements), the main-KV commit writes K and V rows
// with the same row store, and the e4m3 q-store commit packs the query to
// e4m3 with unit scale, saturating (the pack_q_e4m3 commit: beyond +-448 and
// inf saturate, NaN stays NaN).
//
// One wave stores one 128-element row: lane l owns elements 2l and 2l+1, so a
// 32-element group is 16 lanes and its amax is a 16-lane reduction; the wave
// writes the row's 64 data bytes (one per lane) and one dword of 4 scales.
#include "common.hpp"
#include "launch.hpp"
#include "rowstore.hpp"

namespace mxs {

template <int FMT>
__global__ __launch_bounds__(256) void k_row_store(const float *__restrict__ rows, int64_t n,
                                                   const int64_t *__restrict__ slots,
                                                   uint8_t *__restrict__ pages, int32_t num_pages) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int64_t slot = slots[r];
  if (slot < 0 || slot >= (int64_t)num_pages * kTokens) return;
  const float2 x = reinterpret_cast<const float2 *>(rows + r * kDim)[lane];
  const int64_t page = slot / kTokens;
  const int tok = (int)(slot % kTokens);
  if (FMT == 0)
    mx_store_row(x, pages + page * kMxPageBytes, tok, lane);
  else
    f8_store_row(x, pages + page * kF8PageBytes, tok, lane);
}

__global__ __launch_bounds__(256) void k_pack_q(const void *__restrict__ q, int q_dtype, int64_t n,
                                                uint8_t *__restrict__ q8) {
  pack_q4(q, q_dtype, n, q8, ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4);
}

hipError_t launch_row_store(int format, const float *rows, int64_t n, const int64_t *slots,
                            uint8_t *pages, int32_t num_pages, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 3) / 4));
  if (format == 0)
    hipLaunchKernelGGL(k_row_store<0>, grid, dim3(256), 0, s, rows, n, slots, pages, num_pages);
  else
    hipLaunchKernelGGL(k_row_store<1>, grid, dim3(256), 0, s, rows, n, slots, pages, num_pages);
  return hipGetLastError();
}

hipError_t launch_pack_q(const void *q, int q_dtype, int64_t n, uint8_t *q8, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 1023) / 1024));
  hipLaunchKernelGGL(k_pack_q, grid, dim3(256), 0, s, q, q_dtype, n, q8);
  return hipGetLastError();
}

}  // namespace mxs
