// Log-sum-exp merge of split partials for one (query row, head), one wave
// (ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches", commit
// message of the MXFP4 main-KV commit: the merge consumes sp_o / sp_m / sp_l).
//   M = max_p m_p;  L = sum_p l_p e^(m_p - M);  O = sum_p o_p e^(m_p - M) / L;
//   lse = M + ln L.  Empty partitions (m_p = -inf) weigh nothing.
// Lane p < P reads partition p's (m, l); each lane owns two output elements.
#pragma once

#include "common.hpp"

namespace mxs {

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
  a0 *= inv;
  a1 *= inv;
  const uint32_t u0 = f2u(a0), u1 = f2u(a1);
  const uint32_t b0 = (u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16;   // round to nearest even
  const uint32_t b1 = (u1 + 0x7FFFu + ((u1 >> 16) & 1u)) >> 16;
  reinterpret_cast<uint32_t *>(out + r * kDim)[lane] = b0 | (b1 << 16);
  if (lse && lane == 0) lse[r] = Lp > 0.0f ? M + __logf(Lp) : NEG_INF;
}

}  // namespace mxs
