// Row store and q store as stand-alone launches, and the store launch of a
// step that reuses an earlier layer's block selection (the full decode step
// does its stores inside its scorer launch).
//
// ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches": the
// MXFP4 index-cache commit writes each index-key row into an 8704 B page
// (e8m0 group scale, e2m1 elements), the main-KV commit writes K and V rows
// with the same row store, and the e4m3 q-store commit packs the query to
// e4m3 with unit scale, saturating (the pack_q_e4m3 commit: beyond +-448 and
// inf saturate, NaN stays NaN). NVFP4 rows follow the reading stated in
// rowstore.hpp (nv_quant_row).
//
// One wave stores one 128-element row: lane l owns elements 2l and 2l+1, so a
// 32-element group is 16 lanes and its amax is a 16-lane reduction; the wave
// writes the row's 64 data bytes (one per lane) and one dword of 4 scales.
#include <algorithm>

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
  store_row(FMT, x, pages, slot / kTokens, (int)(slot % kTokens), lane);
}

__global__ __launch_bounds__(256) void k_pack_q(const void *__restrict__ q, int q_dtype, int64_t n,
                                                uint8_t *__restrict__ q8) {
  pack_q4(q, q_dtype, n, q8, ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4);
}

// The stores of a step that reuses an earlier layer's block selection (the
// device code is reuse_store_wg in rowstore.hpp).
__global__ __launch_bounds__(256) void k_reuse_store(CacheView c, const float *__restrict__ k_new,
                                                     const float *__restrict__ v_new, const void *__restrict__ q,
                                                     int q_dtype, int H, uint8_t *__restrict__ q8,
                                                     uint64_t *__restrict__ counters, int q_rows) {
  reuse_store_wg<false>(c, k_new, v_new, q, q_dtype, H, q8, counters, q_rows, blockIdx.x);
}

__global__ __launch_bounds__(256) void k_zero(uint32_t *__restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero(uint32_t *p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_reuse_store(const CacheView &c, const float *k_new, const float *v_new, const void *q, int q_dtype,
                              int32_t H, uint8_t *q8, uint64_t *counters, int32_t B, int32_t q_rows, hipStream_t s) {
  if (B * q_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_reuse_store, dim3((unsigned)(B * q_rows)), dim3(256), 0, s, c, k_new, v_new, q, q_dtype, H, q8,
                     counters, q_rows);
  return hipGetLastError();
}

hipError_t launch_row_store(int format, const float *rows, int64_t n, const int64_t *slots,
                            uint8_t *pages, int32_t num_pages, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 3) / 4));
  if (format == 0)
    hipLaunchKernelGGL(k_row_store<0>, grid, dim3(256), 0, s, rows, n, slots, pages, num_pages);
  else if (format == 1)
    hipLaunchKernelGGL(k_row_store<1>, grid, dim3(256), 0, s, rows, n, slots, pages, num_pages);
  else
    hipLaunchKernelGGL(k_row_store<2>, grid, dim3(256), 0, s, rows, n, slots, pages, num_pages);
  return hipGetLastError();
}

hipError_t launch_pack_q(const void *q, int q_dtype, int64_t n, uint8_t *q8, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 1023) / 1024));
  hipLaunchKernelGGL(k_pack_q, grid, dim3(256), 0, s, q, q_dtype, n, q8);
  return hipGetLastError();
}

}  // namespace mxs
