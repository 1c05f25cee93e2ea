// Row store and q store device functions, shared by the stand-alone store
// kernels and the index scorer (which stores the step's new rows itself).
//
// ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches": the
// MXFP4 index-cache commit writes each index-key row into an 8704 B page
// (e8m0 group scale, e2m1 elements), the main-KV commit writes K and V rows
// with the same row store, and the e4m3 q-store commit packs the query to
// e4m3 with unit scale, saturating. NVFP4 rows (named in ATOM PR #2686,
// timeline entry #2744) follow the reading stated at nv_quant_row.
//
// One wave stores one 128-element row: lane l owns elements 2l and 2l+1, so a
// 32-element group is 16 lanes and its amax is a 16-lane reduction; the wave
// writes the row's 64 data bytes (one per lane) and one dword of 4 scales.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mxs {

// Quantize one fp32 row, this wave's lane owning x = elements 2l, 2l+1: the
// lane's code byte (low nibble element 2l) and the e8m0 scale byte of its
// 32-element group (lanes 16 g .. 16 g + 15 hold group g).
__device__ __forceinline__ void mx_quant_row(float2 x, uint32_t &code, uint32_t &sb) {
  uint32_t a = max(f2u(x.x) & 0x7FFFFFFFu, f2u(x.y) & 0x7FFFFFFFu);   // |.| bits order like values
  a = max(a, xor_lane<1>(a));                                          // the 16-lane group's max
  a = max(a, xor_lane<2>(a));
  a = max(a, xor_lane<4>(a));
  a = max(a, xor_lane<8>(a));
  sb = mx_scale_byte(a);
  const float inv = mx_inv_scale(sb);
  code = e2m1_code(x.x * inv) | (e2m1_code(x.y * inv) << 4);
}

// The four group scale bytes of a quantized row as the page's scale dword
// (group g's byte from lane 16 g), the same in every lane.
__device__ __forceinline__ uint32_t mx_scale_word(uint32_t sb) {
  return (uint32_t)__builtin_amdgcn_readlane((int)sb, 0) | ((uint32_t)__builtin_amdgcn_readlane((int)sb, 16) << 8) |
         ((uint32_t)__builtin_amdgcn_readlane((int)sb, 32) << 16) |
         ((uint32_t)__builtin_amdgcn_readlane((int)sb, 48) << 24);
}

// The quantized row into token `tok` of the MXFP4 page at `page` (COH: see st_u8).
template <bool COH = false>
__device__ __forceinline__ void mx_write_row(uint32_t code, uint32_t sb, uint8_t *page, int tok, int lane) {
  st_u8<COH>(page + 64 * tok + lane, code);
  const uint32_t word = mx_scale_word(sb);
  if (lane == 0) st_u32<COH>(reinterpret_cast<uint32_t *>(page + kMxScaleOff + 4 * tok), word);
}

template <bool COH = false>
__device__ __forceinline__ void mx_store_row(float2 x, uint8_t *page, int tok, int lane) {
  uint32_t code, sb;
  mx_quant_row(x, code, sb);
  mx_write_row<COH>(code, sb, page, tok, lane);
}

// FP8 per-token row: scale = fp32(amax / 448) (1 for an all-zero row),
// code = e4m3(fp32(x / scale)); IEEE division on both. codes: the lane's two
// code bytes (element 2l in the low byte).
__device__ __forceinline__ void f8_quant_row(float2 x, uint32_t &codes, float &scale) {
  uint32_t a = max(f2u(x.x) & 0x7FFFFFFFu, f2u(x.y) & 0x7FFFFFFFu);
  a = max(a, xor_lane<1>(a));                                          // the row's max
  a = max(a, xor_lane<2>(a));
  a = max(a, xor_lane<4>(a));
  a = max(a, xor_lane<8>(a));
  a = max(a, xor_lane<16>(a));
  a = max(a, xor_lane<32>(a));
  const float amax = u2f(a);
  scale = amax == 0.0f ? 1.0f : amax / 448.0f;
  codes = e4m3_code(x.x / scale) | (e4m3_code(x.y / scale) << 8);
}

template <bool COH = false>
__device__ __forceinline__ void f8_store_row(float2 x, uint8_t *page, int tok, int lane) {
  uint32_t codes;
  float scale;
  f8_quant_row(x, codes, scale);
  st_u16<COH>(reinterpret_cast<uint16_t *>(page + 128 * tok + 2 * lane), codes);
  if (lane == 0) st_f32<COH>(reinterpret_cast<float *>(page + kF8ScaleOff + 4 * tok), scale);
}

// NVFP4 row (e2m1 in 16-element blocks, e4m3 block scales, a per-token fp32
// scale; the public NVFP4 layout with its second-level scale kept per token):
//   S = amax / 2688 (2688 = 6 * 448), 1 for an all-zero row, 2^-149 where the
//   quotient underflows to 0; block b: c_b = e4m3(a_b / (6 S));
//   code = e2m1(x / (e4m3_value(c_b) * S)), 0 where that divisor is 0;
// every step an IEEE fp32 operation. Lane l owns elements 2l, 2l+1 of block
// l / 8. code: the lane's code byte; cb: its block's scale code.
__device__ __forceinline__ void nv_quant_row(float2 x, uint32_t &code, uint32_t &cb, float &S) {
  uint32_t a = max(f2u(x.x) & 0x7FFFFFFFu, f2u(x.y) & 0x7FFFFFFFu);
  a = max(a, xor_lane<1>(a));
  a = max(a, xor_lane<2>(a));
  a = max(a, xor_lane<4>(a));                                          // the 8-lane block's max
  const float ab = u2f(a);
  a = max(a, xor_lane<8>(a));
  a = max(a, xor_lane<16>(a));
  a = max(a, xor_lane<32>(a));                                         // the row's max
  const float amax = u2f(a);
  const float s = amax / 2688.0f;
  S = amax == 0.0f ? 1.0f : (s == 0.0f ? u2f(1u) : s);                 // u2f(1): 2^-149
  cb = e4m3_code(ab / (6.0f * S));
  const float d = e4m3x2_f32(cb).x * S;
  code = d > 0.0f ? (e2m1_code(x.x / d) | (e2m1_code(x.y / d) << 4)) : 0u;
}

// The eight block scale codes of a quantized NVFP4 row as two dwords (block k's
// code from lane 8 k), the same in every lane.
__device__ __forceinline__ uint2 nv_scale_words(uint32_t cb) {
  auto rl = [&](int l) { return (uint32_t)__builtin_amdgcn_readlane((int)cb, l); };
  return make_uint2(rl(0) | (rl(8) << 8) | (rl(16) << 16) | (rl(24) << 24),
                    rl(32) | (rl(40) << 8) | (rl(48) << 16) | (rl(56) << 24));
}

template <bool COH = false>
__device__ __forceinline__ void nv_store_row(float2 x, uint8_t *page, int tok, int lane) {
  uint32_t code, cb;
  float S;
  nv_quant_row(x, code, cb, S);
  st_u8<COH>(page + 64 * tok + lane, code);
  const uint2 w = nv_scale_words(cb);
  if (lane == 0) {
    st_u32<COH>(reinterpret_cast<uint32_t *>(page + kNvBScaleOff + 8 * tok), w.x);
    st_u32<COH>(reinterpret_cast<uint32_t *>(page + kNvBScaleOff + 8 * tok + 4), w.y);
    st_f32<COH>(reinterpret_cast<float *>(page + kNvTScaleOff + 4 * tok), S);
  }
}

// The new row x (this lane: elements 2 lane, 2 lane + 1) into token `tok` of
// the page at `page`, in cache format `fmt`.
template <bool COH = false>
__device__ __forceinline__ void store_row(int fmt, float2 x, uint8_t *pool, int64_t page, int tok, int lane) {
  if (fmt == 0)
    mx_store_row<COH>(x, pool + page * kMxPageBytes, tok, lane);
  else if (fmt == 1)
    f8_store_row<COH>(x, pool + page * kF8PageBytes, tok, lane);
  else
    nv_store_row<COH>(x, pool + page * kNvPageBytes, tok, lane);
}

__device__ __forceinline__ float load_q_elem(const void *q, int q_dtype, int64_t i) {
  if (q_dtype == 1) return u2f((uint32_t)reinterpret_cast<const uint16_t *>(q)[i] << 16);
  return reinterpret_cast<const float *>(q)[i];
}

// Four consecutive elements per thread, all requested before any is used
// (the dtype branch outside the element loop).
__device__ __forceinline__ void pack_q4(const void *q, int q_dtype, int64_t n, uint8_t *q8, int64_t i) {
  if (i >= n) return;
  const int m = (int)min<int64_t>(4, n - i);
  float v[4];
  if (q_dtype == 1) {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(q) + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < m ? u2f((uint32_t)p[e] << 16) : 0.0f;
  } else {
    const float *p = reinterpret_cast<const float *>(q) + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < m ? p[e] : 0.0f;
  }
  if (m == 4 && ((reinterpret_cast<uintptr_t>(q8) + i) & 3) == 0) {
    *reinterpret_cast<uint32_t *>(q8 + i) =
        e4m3_code(v[0]) | (e4m3_code(v[1]) << 8) | (e4m3_code(v[2]) << 16) | (e4m3_code(v[3]) << 24);
  } else {
    for (int e = 0; e < m; ++e) q8[i + e] = (uint8_t)e4m3_code(v[e]);
  }
}

// The stores of a step that reuses an earlier layer's block selection (the
// pages' index_topk_freq schedule: such a layer scores nothing), one
// workgroup per query row (row = b q_rows + j). The workgroup stores the new
// K and V rows of position L_b - q + j (wave 0: K, wave 1: V; skipped when
// that position has no valid page), packs the row's H x 128 query elements
// to e4m3 (waves 2 - 3, when q8 is given) and clears the row's merge counter
// (when counters is given) for the attention that follows. Every load
// that does not depend on another is requested before any result is used:
// the source row goes out with the context length (the page id needs the
// length), and each packing thread requests its 16 query elements at once.
// COH: every store device-coherent (read by other workgroups of the same
// launch once the workgroup has counted itself in).
template <bool COH>
__device__ __forceinline__ void reuse_store_wg(const CacheView &c, const float *__restrict__ k_new,
                                               const float *__restrict__ v_new, const void *__restrict__ q,
                                               int q_dtype, int H, uint8_t *__restrict__ q8,
                                               uint64_t *__restrict__ counters, int q_rows, int row) {
  const int b = row / q_rows, j = row % q_rows;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  if (counters && tid == 0) st_u64<COH>(counters + row, 0ull);
  if (wave < 2) {
    const float *src = wave == 0 ? k_new : v_new;
    if (!src) return;
    const float2 x = reinterpret_cast<const float2 *>(src + (int64_t)row * kDim)[lane];
    const int pos = c.context_lens[b] - q_rows + j;
    if (pos < 0 || pos / kTokens >= c.stride) return;
    const int phys = c.page_table[(int64_t)b * c.stride + pos / kTokens];
    if (phys < 0 || phys >= c.num_pages) return;
    store_row<COH>(c.kv_format, x, wave == 0 ? c.k_pages : c.v_pages, phys, pos % kTokens, lane);
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
    if constexpr (COH) {
#pragma unroll
      for (int k = 0; k < 4; ++k) st_u32<true>(reinterpret_cast<uint32_t *>(q8 + e0) + k, codes[k]);
    } else {
      *reinterpret_cast<u32x4 *>(q8 + e0) = codes;      // q8: the step workspace, 16-byte aligned
    }
  }
}

}  // namespace mxs
