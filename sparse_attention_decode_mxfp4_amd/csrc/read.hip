// Streaming-read ceiling of the index scan: every index page of every
// sequence read once, in page-table order, with plain 16-byte loads folded
// into one word per workgroup. Nothing is widened, multiplied or written (one
// word at most), so its time is how fast this part can deliver the scorer's
// input from HBM: the bound the index scorer is compared with. Its loads take
// the scorer's non-temporal cache policy (4 sequences x 2048 pages: 12.0 us
// against 13.9 us with cached loads). It computes nothing of the method.
#include "common.hpp"
#include "launch.hpp"

namespace mxs {

constexpr int kReadThreads = 256;
constexpr int kReadPages = 4;     // logical pages per workgroup
constexpr int kReadUnroll = 9;    // 16-byte loads in flight per thread: 4 MXFP4 pages = 2176 chunks <= 256 x 9

// grid (sequence, group of kReadPages logical pages); PAGE_BYTES a multiple of 16
template <uint32_t PAGE_BYTES>
__global__ __launch_bounds__(kReadThreads) void k_read_pages(const uint8_t *__restrict__ pages, int32_t num_pages,
                                                             const int32_t *__restrict__ page_table, int32_t stride,
                                                             const int32_t *__restrict__ context_lens,
                                                             uint32_t *__restrict__ sink) {
  __shared__ int32_t s_page[kReadPages];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = context_lens[b];
  const int n_pages = min(stride, L > 0 ? (L + 127) / 128 : 0);
  const int p0 = blockIdx.y * kReadPages, n = min(kReadPages, n_pages - p0);
  if (n <= 0) return;                                  // uniform over the workgroup
  if (tid < n) {
    const int pg = page_table[(size_t)b * stride + p0 + tid];
    s_page[tid] = pg >= 0 && pg < num_pages ? pg : -1;   // out-of-pool entries are not read
  }
  __syncthreads();
  constexpr uint32_t per_page = PAGE_BYTES / 16;
  const uint32_t n_chunks = (uint32_t)n * per_page;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t c0 = tid; c0 < n_chunks; c0 += kReadThreads * kReadUnroll) {
    u32x4 v[kReadUnroll];
    int pg[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {          // the page ids first, then every load at once
      const uint32_t c = c0 + (uint32_t)(u * kReadThreads);
      pg[u] = c < n_chunks ? s_page[c / per_page] : -1;
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {          // a lane with nothing to read loads the pool's first chunk
      const uint32_t c = c0 + (uint32_t)(u * kReadThreads);
      const size_t off = pg[u] >= 0 ? (size_t)pg[u] * PAGE_BYTES + (size_t)(c % per_page) * 16u : 0;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(pages + off));
      if (pg[u] < 0) v[u] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) sink[0] = x;                   // keeps the loads alive; the value carries no meaning
}

hipError_t launch_read_pages(const CacheView &c, int32_t B, uint32_t page_bytes, uint32_t *sink, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)B, (unsigned)((c.stride + kReadPages - 1) / kReadPages));
  if (page_bytes == 8704u)
    hipLaunchKernelGGL(k_read_pages<8704u>, grid, dim3(kReadThreads), 0, s, c.idx_pages, c.num_pages, c.page_table,
                       c.stride, c.context_lens, sink);
  else if (page_bytes == 16896u)
    hipLaunchKernelGGL(k_read_pages<16896u>, grid, dim3(kReadThreads), 0, s, c.idx_pages, c.num_pages, c.page_table,
                       c.stride, c.context_lens, sink);
  else if (page_bytes == 9728u)
    hipLaunchKernelGGL(k_read_pages<9728u>, grid, dim3(kReadThreads), 0, s, c.idx_pages, c.num_pages, c.page_table,
                       c.stride, c.context_lens, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mxs
