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
// pages' index_topk_freq schedule: such a layer scores nothing). Workgroup
// (b, j) stores the new K and V rows of position L_b - q + j (wave 0: K,
// wave 1: V; skipped when that position has no valid page), packs the row's
// H x 128 query elements to e4m3 (waves 2 - 3, when q8 is given) and clears
// the row's merge counter for the attention launch that follows. Every load
// that does not depend on another is requested before any result is used:
// the source row goes out with the context length (the page id needs the
// length), and each packing thread requests its 16 query elements at once.
__global__ __launch_bounds__(256) void k_reuse_store(CacheView c, const float *__restrict__ k_new,
                                                     const float *__restrict__ v_new, const void *__restrict__ q,
                                                     int q_dtype, int H, uint8_t *__restrict__ q8,
                                                     uint32_t *__restrict__ counters, int q_rows) {
  const int row = blockIdx.x, b = row / q_rows, j = row % q_rows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) counters[row] = 0u;
  if (wave < 2) {
    const float *src = wave == 0 ? k_new : v_new;
    if (!src) return;
    const float2 x = reinterpret_cast<const float2 *>(src + (int64_t)row * kDim)[lane];
    const int pos = c.context_lens[b] - q_rows + j;
    if (pos < 0 || pos / kTokens >= c.stride) return;
    const int phys = c.page_table[(int64_t)b * c.stride + pos / kTokens];
    if (phys < 0 || phys >= c.num_pages) return;
    store_row(c.kv_format, x, wave == 0 ? c.k_pages : c.v_pages, phys, pos % kTokens, lane);
  } else if (q8) {
    // elements e0 .. e0 + 15 of the row (H x 128 <= 2048 = 16 x 128 threads);
    // the query is 16-byte aligned, so are the row and each thread's run
    const int t = tid - 128;
    if (16 * t >= H * kDim) return;
    const int64_t e0 = (int64_t)row * H * kDim + 16 * t;
    float v[16];
    if (q_dtype == 1) {                               // bf16: element 2k in the low half of dword k
      const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(q) + e0);
      const u32x4 a0 = p[0], a1 = p[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = u2f(a0[k] << 16);
        v[2 * k + 1] = u2f(a0[k] & 0xFFFF0000u);
        v[8 + 2 * k] = u2f(a1[k] << 16);
        v[8 + 2 * k + 1] = u2f(a1[k] & 0xFFFF0000u);
      }
    } else {
      const u32x4 *p = reinterpret_cast<const u32x4 *>(static_cast<const float *>(q) + e0);
      u32x4 a[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = p[k];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = u2f(a[k >> 2][k & 3]);
    }
    u32x4 codes;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      codes[k] = e4m3_code(v[4 * k]) | (e4m3_code(v[4 * k + 1]) << 8) | (e4m3_code(v[4 * k + 2]) << 16) |
                 (e4m3_code(v[4 * k + 3]) << 24);
    *reinterpret_cast<u32x4 *>(q8 + e0) = codes;        // q8: the step workspace, 16-byte aligned
  }
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
                              int32_t H, uint8_t *q8, uint32_t *counters, int32_t B, int32_t q_rows, hipStream_t s) {
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
