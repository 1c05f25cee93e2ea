// Row store and q store: the step's first kernel.
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

namespace mxs {

// Quantize one fp32 row (this wave's lane owns x = elements 2l, 2l+1) into
// token `tok` of the MXFP4 page at `page`.
__device__ __forceinline__ void mx_store_row(float2 x, uint8_t *page, int tok, int lane) {
  uint32_t a = max(f2u(x.x) & 0x7FFFFFFFu, f2u(x.y) & 0x7FFFFFFFu);   // |.| bits order like values
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  a = max(a, (uint32_t)__shfl_xor((int)a, 2));
  a = max(a, (uint32_t)__shfl_xor((int)a, 4));
  a = max(a, (uint32_t)__shfl_xor((int)a, 8));
  const uint32_t sb = mx_scale_byte(a);
  const float inv = mx_inv_scale(sb);
  const uint32_t c0 = e2m1_code(x.x * inv);
  const uint32_t c1 = e2m1_code(x.y * inv);
  page[64 * tok + lane] = (uint8_t)(c0 | (c1 << 4));
  const uint32_t s1 = (uint32_t)__shfl((int)sb, 16);
  const uint32_t s2 = (uint32_t)__shfl((int)sb, 32);
  const uint32_t s3 = (uint32_t)__shfl((int)sb, 48);
  if (lane == 0)
    *reinterpret_cast<uint32_t *>(page + kMxScaleOff + 4 * tok) = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

// FP8 per-token row: scale = fp32(amax / 448) (1 for an all-zero row),
// code = e4m3(fp32(x / scale)); IEEE division on both.
__device__ __forceinline__ void f8_store_row(float2 x, uint8_t *page, int tok, int lane) {
  uint32_t a = max(f2u(x.x) & 0x7FFFFFFFu, f2u(x.y) & 0x7FFFFFFFu);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) a = max(a, (uint32_t)__shfl_xor((int)a, o));
  const float amax = u2f(a);
  const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;
  const uint32_t c0 = e4m3_code(x.x / scale);
  const uint32_t c1 = e4m3_code(x.y / scale);
  *reinterpret_cast<uint16_t *>(page + 128 * tok + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) *reinterpret_cast<float *>(page + kF8ScaleOff + 4 * tok) = scale;
}

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

__device__ __forceinline__ float load_q_elem(const void *q, int q_dtype, int64_t i) {
  if (q_dtype == 1) return u2f((uint32_t)reinterpret_cast<const uint16_t *>(q)[i] << 16);
  return reinterpret_cast<const float *>(q)[i];
}

// Four consecutive elements per thread.
__device__ __forceinline__ void pack_q4(const void *q, int q_dtype, int64_t n, uint8_t *q8, int64_t i) {
  if (i >= n) return;
  if (i + 4 <= n && ((reinterpret_cast<uintptr_t>(q8) + i) & 3) == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w |= e4m3_code(load_q_elem(q, q_dtype, i + e)) << (8 * e);
    *reinterpret_cast<uint32_t *>(q8 + i) = w;
  } else {
    for (int e = 0; e < 4 && i + e < n; ++e) q8[i + e] = (uint8_t)e4m3_code(load_q_elem(q, q_dtype, i + e));
  }
}

__global__ __launch_bounds__(256) void k_pack_q(const void *__restrict__ q, int q_dtype, int64_t n,
                                                uint8_t *__restrict__ q8) {
  pack_q4(q, q_dtype, n, q8, ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4);
}

// decode_step's store: blockIdx.y = 0 / 1 / 2 stores the step's new K / V /
// index rows (row j of sequence b goes to position L_b - q + j); 3 packs q.
__global__ __launch_bounds__(256) void k_step_store(CacheView c, const float *__restrict__ k_new,
                                                    const float *__restrict__ v_new,
                                                    const float *__restrict__ idx_new, int32_t B,
                                                    int32_t q, const void *__restrict__ q_att,
                                                    int q_dtype, int64_t q_elems,
                                                    uint8_t *__restrict__ q8) {
  if (blockIdx.y == 3) {
    if (q8) pack_q4(q_att, q_dtype, q_elems, q8, ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4);
    return;
  }
  const float *src = blockIdx.y == 0 ? k_new : (blockIdx.y == 1 ? v_new : idx_new);
  if (!src) return;
  uint8_t *pool = blockIdx.y == 0 ? c.k_pages : (blockIdx.y == 1 ? c.v_pages : c.idx_pages);
  const int fmt = blockIdx.y == 2 ? c.idx_format : c.kv_format;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= B * q) return;
  const int b = r / q, j = r % q;
  const int t = c.context_lens[b] - q + j;
  if (t < 0 || t / kTokens >= c.stride) return;
  const int page = c.page_table[(int64_t)b * c.stride + t / kTokens];
  if (page < 0 || page >= c.num_pages) return;
  const float2 x = reinterpret_cast<const float2 *>(src + (int64_t)r * kDim)[lane];
  if (fmt == 0)
    mx_store_row(x, pool + (int64_t)page * kMxPageBytes, t % kTokens, lane);
  else
    f8_store_row(x, pool + (int64_t)page * kF8PageBytes, t % kTokens, lane);
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

hipError_t launch_step_store(const CacheView &c, const float *k_new, const float *v_new,
                             const float *idx_new, int32_t B, int32_t q, const void *q_att,
                             int q_dtype, int64_t q_elems, uint8_t *q8, hipStream_t s) {
  const int64_t row_blocks = ((int64_t)B * q + 3) / 4;
  const int64_t q_blocks = (q_elems + 1023) / 1024;
  const dim3 grid((unsigned)(row_blocks > q_blocks ? row_blocks : q_blocks), 4);
  hipLaunchKernelGGL(k_step_store, grid, dim3(256), 0, s, c, k_new, v_new, idx_new, B, q, q_att,
                     q_dtype, q_elems, q8);
  return hipGetLastError();
}

}  // namespace mxs
