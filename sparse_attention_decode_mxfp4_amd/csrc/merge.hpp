// Log-sum-exp merge of split partials (ATOM PR #2812, "Mono decode over the
// MXFP4 KV and index caches", commit message of the MXFP4 main-KV commit: the
// merge consumes sp_o / sp_m / sp_l):
//   M = max_p m_p;  L = sum_p l_p e^(m_p - M);  O = sum_p o_p e^(m_p - M) / L;
//   lse = M + ln L.  Empty partitions (m_p = -inf) weigh nothing.
// merge_one: one (query row, head) per wave (the stand-alone merge kernel);
// lane p < P reads partition p's (m, l), each lane owns two output elements.
// merge_row: one query row per workgroup (the decode step's in-launch merge;
// COH: the partials are read device-coherently, else through this XCD's L2).
#pragma once

#include "common.hpp"

namespace mxs {

// Device-coherent 16-byte partial traffic for the decode step's in-launch
// merge: buffer loads / stores with the sc1 cache-policy bit (the bit an
// agent-scope relaxed atomic load or store carries), through a descriptor
// over one query row's partials (bounds-checked by the hardware).
constexpr int kCoherentBits = 16;                     // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float *base, int32_t n_floats) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, n_floats * 4, 0x00020000);
}
// (the builtins move raw 32-bit words: every value crosses as its bits)
__device__ __forceinline__ f32x4 load4_coherent(__amdgpu_buffer_rsrc_t rs, int32_t float_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, float_off * 4, 0, kCoherentBits));
}
__device__ __forceinline__ float load1_coherent(__amdgpu_buffer_rsrc_t rs, int32_t float_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, float_off * 4, 0, kCoherentBits));
}
// Loads of another workgroup's partials: device-coherent (COH, sc1: past
// this XCD's L2, for data written on any XCD) or plain (through this XCD's L2:
// for data written on the same XCD, never loaded into this CU's L1 before).
template <bool COH>
__device__ __forceinline__ f32x4 load4_partial(__amdgpu_buffer_rsrc_t rs, int32_t float_off) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(rs, float_off * 4, 0, COH ? kCoherentBits : 0));
}
template <bool COH>
__device__ __forceinline__ float load1_partial(__amdgpu_buffer_rsrc_t rs, int32_t float_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, float_off * 4, 0, COH ? kCoherentBits : 0));
}
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t rs, int32_t float_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, float_off * 4, 0, kCoherentBits);
}

__device__ __forceinline__ void merge_one(const float *__restrict__ sp_m, const float *__restrict__ sp_l,
                                          const float *__restrict__ sp_o, int64_t r, int32_t P, int lane,
                                          uint16_t *__restrict__ out, float *__restrict__ lse) {
  const float NEG_INF = -__builtin_inff();
  const float mraw = sp_m[r * P + min(lane, P - 1)];
  const float lraw = sp_l[r * P + min(lane, P - 1)];
  const float2 *po = reinterpret_cast<const float2 *>(sp_o + r * P * kDim) + lane;
  float2 v[8];                                  // the first 8 partitions' outputs, requested with (m, l)
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = po[min(u, P - 1) * (kDim / 2)];   // clamped: no branch
  const float mp = lane < P ? mraw : NEG_INF;
  float M = mp;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float wp = (lane < P && mp != NEG_INF) ? __expf(mp - M) : 0.0f;
  float Lp = lane < P ? lraw * wp : 0.0f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) Lp += __shfl_xor(Lp, o);
  const float inv = Lp > 0.0f ? 1.0f / Lp : 0.0f;
  float a0 = 0.f, a1 = 0.f;
  for (int p0 = 0; p0 < P; p0 += 8) {
    if (p0 > 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = po[min(p0 + u, P - 1) * (kDim / 2)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wq = __shfl(wp, p0 + u < P ? p0 + u : 0);
      if (p0 + u < P && wq != 0.0f) {
        a0 += wq * v[u].x;
        a1 += wq * v[u].y;
      }
    }
  }
  const bf16x2 o = {(__bf16)(a0 * inv), (__bf16)(a1 * inv)};     // round to nearest even (v_cvt_pk_bf16_f32)
  reinterpret_cast<uint32_t *>(out + r * kDim)[lane] = bf16x2_bits(o);
  if (lse && lane == 0) lse[r] = Lp > 0.0f ? M + __logf(Lp) : NEG_INF;
}

// One query row (H <= 16 heads) merged by a 256-thread workgroup: thread t
// takes head t / 16 and output elements 8 (t % 16) .. + 7. Every partition's
// (m, l) and the thread's 8 elements of every partition's O are requested at
// once, 8 partitions per round (more partitions fold in with an online
// rescale), so the merge costs one memory round trip for P <= 8. The
// partials were written by other workgroups of the same launch (device-
// coherent stores), so every load is device-coherent too.
template <bool COH>
__device__ __forceinline__ void merge_row(const float *__restrict__ sp_m, const float *__restrict__ sp_l,
                                          const float *__restrict__ sp_o, int64_t row, int32_t H, int32_t P,
                                          int32_t mls, uint16_t *__restrict__ out, float *__restrict__ lse) {
  const float NEG_INF = -__builtin_inff();
  const int t = threadIdx.x, h = t >> 4, e0 = 8 * (t & 15);
  if (h >= H) return;
  const int64_t r = row * H + h;
  float M = NEG_INF, Lsum = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const __amdgpu_buffer_rsrc_t ro = row_rsrc(sp_o + row * H * P * kDim, H * P * kDim);
  // (m, l) of 4 partitions per 16-byte load when P is a multiple of 4 (the
  // row's (m, l) arrays, mls floats apart, are then 16-byte aligned); reads past
  // the row's last head return 0 (descriptor bound) and, like every u >= P - p0,
  // weigh nothing
  const bool ml4 = (P & 3) == 0 && (mls & 3) == 0;
  const __amdgpu_buffer_rsrc_t rm = row_rsrc(sp_m + row * mls, H * P), rl = row_rsrc(sp_l + row * mls, H * P);
  for (int p0 = 0; p0 < P; p0 += 8) {
    float m[8], l[8];
    f32x4 o[8][2];
    if (ml4) {
      const f32x4 m0 = load4_partial<COH>(rm, h * P + p0), m1 = load4_partial<COH>(rm, h * P + p0 + 4);
      const f32x4 l0 = load4_partial<COH>(rl, h * P + p0), l1 = load4_partial<COH>(rl, h * P + p0 + 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m[u] = m0[u];
        m[u + 4] = m1[u];
        l[u] = l0[u];
        l[u + 4] = l1[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) {               // clamped, unconditional
        const int pp = min(p0 + u, P - 1);
        m[u] = load1_partial<COH>(rm, h * P + pp);
        l[u] = load1_partial<COH>(rl, h * P + pp);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {                 // clamped, unconditional; u >= P - p0 weigh nothing
      const int pp = min(p0 + u, P - 1);
      const int32_t off = (h * P + pp) * kDim + e0;
#pragma unroll
      for (int k = 0; k < 2; ++k) o[u][k] = load4_partial<COH>(ro, off + 4 * k);
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) Mc = (p0 + u < P) ? fmaxf(Mc, m[u]) : Mc;
    const float a = (M == NEG_INF) ? 0.0f : __expf(M - Mc);    // rescale what is folded in so far
    Lsum *= a;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= a;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wu = (p0 + u < P && m[u] != NEG_INF) ? __expf(m[u] - Mc) : 0.0f;
      if (wu != 0.0f) {
        Lsum += l[u] * wu;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wu * o[u][e >> 2][e & 3];
      }
    }
    M = Mc;
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  u32x4 packed;
#pragma unroll
  for (int k = 0; k < 4; ++k) {                   // round to nearest even (v_cvt_pk_bf16_f32)
    const bf16x2 v = {(__bf16)(acc[2 * k] * inv), (__bf16)(acc[2 * k + 1] * inv)};
    packed[k] = bf16x2_bits(v);
  }
  uint16_t *const dst = out + r * kDim + e0;      // out: at least 4-byte aligned
  if ((reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    *reinterpret_cast<u32x4 *>(dst) = packed;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) reinterpret_cast<uint32_t *>(dst)[k] = packed[k];
  }
  if (lse && (t & 15) == 0) lse[r] = Lsum > 0.0f ? M + __logf(Lsum) : NEG_INF;
}

}  // namespace mxs
