// Split-KV sparse attention over the selected pages.
//
// ATOM PR #2812, "Mono decode over the MXFP4 KV and index caches", commit
// message of the MXFP4 main-KV commit: the split stage reads the K and V pages
// of the sparse (block) table — one selected block is one 128-token page —
// and writes per-partition partials sp_o / sp_m / sp_l for a merge. There, QK
// is one MX-scaled 16x16x128 MFMA (K fp4 with its e8m0 group scale against
// the e4m3 query) and PV a bf16 MFMA over V widened to bf16. This kernel keeps
// the matrix-core split of work but lays the operands out its own way:
//
// * Workgroup = (partition p, query row j, sequence b), 4 waves. Partition p
//   owns block-table slots [p c, min((p+1) c, topk)), c = ceil(topk / P); wave
//   w takes every 4th of them, keeps an online softmax (m, l, O) for the 16
//   heads, and the 4 waves merge through LDS into one partial. A wave's token
//   range is a whole block, or half a block when a partition owns at most two
//   blocks (step_tiles: waves in pairs, so that all 4 waves work; with whole
//   blocks two of them would idle). (Half blocks for 8-wave workgroups
//   measured slower on MI355X: the 8-wave selection and merge lose more at
//   their barriers than the halved block work gains.)
// * QK: D[token][head] = K[token][:] . q[head][:] on v_mfma_f32_16x16x32_bf16.
//   Lane 16 kg + n loads token n's group kg — 16 bytes and one scale byte, the
//   same coalesced pattern as the index scorer — and widens it to bf16 with
//   the group scale (exact); the e4m3 query is widened to bf16 once (exact).
//   The pages run QK on the MX-scaled fp4 x fp8 MFMA instead; measured on
//   gfx950, that instruction rounds a 32-product block to ~14 bits relative
//   to its largest product, which a saturated (+-448) query element turns
//   into softmax errors beyond the parity bound, so the exact-product bf16
//   MFMA with fp32 accumulation is used here. Tokens past the row's position
//   are zeroed before the MFMA and masked after it, so NaN-poisoned tails
//   never reach an accumulator.
// * PV: O[head][d] += P[head][token] V[token][d] on v_mfma_f32_16x16x32_bf16.
//   The QK result leaves each lane P for head n and tokens 4 kg + i of each
//   16-token tile, which is directly a valid A operand once the k-step's token
//   order is taken as {32 s + 4 kg + i, 32 s + 16 + 4 kg + i}. The output
//   column order is permuted, d = 8 n + dt for d-tile dt, so that the B
//   operand of lane (n, kg) needs, per token, the 8 consecutive codes
//   d = 8 n .. 8 n + 7: one 4-byte load per token. Each byte widens to two
//   bf16 (v_cvt_scalef32_pk_bf16_fp4 with the token's group scale) and a 2x2
//   half-word transpose forms the MFMA operands; no LDS round trip.
// * FP8 KV (e4m3 codes, per-token fp32 scale, bf16 query): QK on the bf16
//   MFMA with the codes widened exactly to bf16 and the token scale applied to
//   the dot product; PV folds the token scale into P.
// * NVFP4 KV (e2m1 in 16-element blocks with e4m3 block scales, per-token fp32
//   scale, bf16 query): the MXFP4 lane layout, the codes widened times their
//   block scale (exact): K to f16 for QK on the f16 MFMA against the query
//   scaled per head into f16 (query_operands_f16), V to bf16 for PV; the token
//   scale handled as for FP8.
#include "common.hpp"
#include "launch.hpp"
#include "topk.hpp"
#include "merge.hpp"
#include "mxsparse.h"
#include "score.hpp"
#include "rowstore.hpp"

namespace mxs {

constexpr int kAttnWaves = 4;    // the stand-alone split stage
constexpr int kStepWaves = 4;    // the decode step's attention launch

// 16-token tiles per wave's token range in the attention launches: whole
// blocks (8), or half blocks (4) when a partition owns at most two blocks, so
// that its 4 waves all work (two waves per block). Measured on MI355X at the
// default partition counts (step, same session): top-k 16 over 4 x 4 FP8 rows
// 15.2 against 16.2 us; top-k 16 over 4 x 8 NVFP4 rows (8 partitions) 19.1
// against 20.3 us with whole blocks at 4 partitions; the MXFP4 65K workload
// 18.1 against 18.4 us. With more than two blocks per partition whole blocks
// win (top-k 32 over 4 x 8 rows: 32.5 us against 33.2 us for half blocks).
constexpr int step_tiles(int topk, int P) { return (topk + P - 1) / P <= 2 ? 4 : 8; }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Half-word pairs of two dwords (v_perm_b32): the low halves of x and y, and
// the high halves, x's in the low half of the result.
__device__ __forceinline__ uint32_t lo_pair(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); }
// fp32 value of an e8m0 scale byte for the cvt_scalef32 instructions:
// byte << 23 is 2^(byte - 127) for byte >= 1, and byte 0 takes 0x400000 = 2^-127.
__device__ __forceinline__ float e8m0_scale(uint32_t byte) { return u2f(max(byte << 23, 0x00400000u)); }

// The operands of a wave's token range of one block (NT 16-token tiles from
// token toff of the page: the whole page, NT = 8, or one half, NT = 4), as this
// lane loads them (all requested before any math).
//  K: tile nt -> token toff + 16 nt + n; MXFP4: 16 bytes of group kg + its scale
//     byte; FP8: 32 bytes (elements 32 kg .. + 31) + 4 token scales (tokens
//     toff + 16 nt + 4 kg + i).
//  V: k-step s -> the 8 tokens toff + te(s, e); MXFP4: 4 bytes (codes 8 n ..
//     8 n + 7) per token + the scale dwords of the two 4-token runs; FP8: 8
//     bytes per token + the fp32 scales of the two runs.
//  NVFP4: K as MXFP4 with the two block scale codes of group kg (kb) and the
//     fp32 scales of tokens toff + 16 nt + 4 kg + i (ks, as FP8); V as MXFP4
//     with, per token, the dword holding the scale code of block n / 2 (vb)
//     and the fp32 scales of the two runs (vs, as FP8).
template <int FMT, int NT> struct BlockRegs;
template <int NT> struct BlockRegs<0, NT> { u32x4 k[NT]; uint32_t ks[NT]; uint32_t v[NT / 2][8]; u32x4 vs[NT / 2][2]; };
template <int NT> struct BlockRegs<1, NT> { u32x4 k[NT][2]; f32x4 ks[NT]; uint2 v[NT / 2][8]; f32x4 vs[NT / 2][2]; };
template <int NT> struct BlockRegs<2, NT> {
  u32x4 k[NT]; uint32_t kb[NT]; f32x4 ks[NT]; uint32_t v[NT / 2][8]; uint32_t vb[NT / 2][8]; f32x4 vs[NT / 2][2];
};

// token of element e of the lane's k-group in PV k-step s
__device__ __forceinline__ int pv_token(int s, int kg, int e) { return 32 * s + (e < 4 ? 4 * kg + e : 16 + 4 * kg + e - 4); }

template <int FMT, int NT>
__device__ __forceinline__ void load_block(BlockRegs<FMT, NT> &r, const uint8_t *kp, const uint8_t *vp, int toff, int n,
                                           int kg) {
  if constexpr (FMT == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tok = toff + 16 * nt + n;
      r.k[nt] = *reinterpret_cast<const u32x4 *>(kp + 64 * tok + 16 * kg);
      r.ks[nt] = kp[kMxScaleOff + 4 * tok + kg];
    }
#pragma unroll
    for (int s = 0; s < NT / 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        r.v[s][e] = *reinterpret_cast<const uint32_t *>(vp + 64 * (toff + pv_token(s, kg, e)) + 4 * n);
      r.vs[s][0] = *reinterpret_cast<const u32x4 *>(vp + kMxScaleOff + 4 * (toff + pv_token(s, kg, 0)));
      r.vs[s][1] = *reinterpret_cast<const u32x4 *>(vp + kMxScaleOff + 4 * (toff + pv_token(s, kg, 4)));
    }
  } else if constexpr (FMT == 2) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tok = toff + 16 * nt + n;
      r.k[nt] = *reinterpret_cast<const u32x4 *>(kp + 64 * tok + 16 * kg);
      r.kb[nt] = *reinterpret_cast<const uint16_t *>(kp + kNvBScaleOff + 8 * tok + 2 * kg);
      r.ks[nt] = *reinterpret_cast<const f32x4 *>(kp + kNvTScaleOff + 4 * (toff + 16 * nt + 4 * kg));
    }
    // one lane base each for the codes and the block scale dwords, constant
    // offsets from there (computed per load, the block scale addresses took
    // enough registers to spill)
    const uint8_t *vcode = vp + 64 * (toff + 4 * kg) + 4 * n;
    const uint8_t *vbsc = vp + kNvBScaleOff + 8 * (toff + 4 * kg) + 4 * (n >> 3);
#pragma unroll
    for (int s = 0; s < NT / 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dt = pv_token(s, 0, e);              // the token's offset from toff + 4 kg
        r.v[s][e] = *reinterpret_cast<const uint32_t *>(vcode + 64 * dt);
        r.vb[s][e] = *reinterpret_cast<const uint32_t *>(vbsc + 8 * dt);
      }
      r.vs[s][0] = *reinterpret_cast<const f32x4 *>(vp + kNvTScaleOff + 4 * (toff + pv_token(s, kg, 0)));
      r.vs[s][1] = *reinterpret_cast<const f32x4 *>(vp + kNvTScaleOff + 4 * (toff + pv_token(s, kg, 4)));
    }
  } else {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int tok = toff + 16 * nt + n;
      r.k[nt][0] = *reinterpret_cast<const u32x4 *>(kp + 128 * tok + 32 * kg);
      r.k[nt][1] = *reinterpret_cast<const u32x4 *>(kp + 128 * tok + 32 * kg + 16);
      r.ks[nt] = *reinterpret_cast<const f32x4 *>(kp + kF8ScaleOff + 4 * (toff + 16 * nt + 4 * kg));
    }
#pragma unroll
    for (int s = 0; s < NT / 2; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        r.v[s][e] = *reinterpret_cast<const uint2 *>(vp + 128 * (toff + pv_token(s, kg, e)) + 8 * n);
      r.vs[s][0] = *reinterpret_cast<const f32x4 *>(vp + kF8ScaleOff + 4 * (toff + pv_token(s, kg, 0)));
      r.vs[s][1] = *reinterpret_cast<const f32x4 *>(vp + kF8ScaleOff + 4 * (toff + pv_token(s, kg, 4)));
    }
  }
}

// The lane's query elements for QK, as loaded: head n, elements 32 kg + 8 s
// .. + 7 for k-step s (the order of the key groups each lane loads); e4m3
// codes with an MXFP4 cache, bf16 with an FP8 or NVFP4 cache. Heads >= H load
// head 0 (unconditional loads) and are zeroed when the operands are formed.
template <int FMT> struct QueryRegs { u32x4 c[4]; };
template <> struct QueryRegs<0> { uint2 c[4]; };

template <int FMT, bool COH = false>
__device__ __forceinline__ void load_query(const void *__restrict__ qv, int row, int H, int n, int kg,
                                           QueryRegs<FMT> &q) {
  const int64_t base = ((int64_t)row * H + (n < H ? n : 0)) * kDim + 32 * kg;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (FMT == 0) {
      const uint8_t *src = reinterpret_cast<const uint8_t *>(qv) + base + 8 * s;
      if constexpr (COH) {                         // written earlier in the same launch (device-coherent)
        const uint64_t x = __hip_atomic_load(reinterpret_cast<const uint64_t *>(src), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        q.c[s] = make_uint2((uint32_t)x, (uint32_t)(x >> 32));
      } else {
        q.c[s] = *reinterpret_cast<const uint2 *>(src);
      }
    } else {
      static_assert(!COH || FMT == 0, "the single-launch step packs an e4m3 query");
      q.c[s] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(qv) + base + 8 * s);
    }
  }
}

// The lane's query elements as load_query takes them (head n, elements
// 32 kg + 8 s .. + 7), from the caller's fp32 or bf16 query, for a launch that
// rounds the query to e4m3 itself instead of reading packed codes.
struct RawQuery {
  u32x4 v[8];                                      // fp32: k-step s in v[2 s], v[2 s + 1]; bf16: in v[s]
};
__device__ __forceinline__ void load_query_raw(const void *__restrict__ qv, int q_dtype, int row, int H, int n, int kg,
                                               RawQuery &r) {
  const int64_t base = ((int64_t)row * H + (n < H ? n : 0)) * kDim + 32 * kg;
  if (q_dtype == 1) {
#pragma unroll
    for (int s = 0; s < 4; ++s) r.v[s] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(qv) + base + 8 * s);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) r.v[k] = *reinterpret_cast<const u32x4 *>(static_cast<const float *>(qv) + base + 4 * k);
  }
}
// Two values as e4m3 codes in bytes 0 and 1 (or 2 and 3, HI) of `old`: the
// saturating e4m3 store's rounding. v_cvt_pk_fp8_f32 rounds to nearest even
// and gives NaN above 464 (checked on MI355X against the software encoder on
// every e4m3 midpoint, its neighbours and the range's ends), so values past
// +-448 are first set to +-448; NaN fails the comparison and stays NaN.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, uint32_t old) {
  a = __builtin_fabsf(a) > 448.0f ? __builtin_copysignf(448.0f, a) : a;
  b = __builtin_fabsf(b) > 448.0f ? __builtin_copysignf(448.0f, b) : b;
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}
__device__ __forceinline__ void round_query_e4m3(const RawQuery &r, int q_dtype, QueryRegs<0> &q) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float x[8];
    if (q_dtype == 1) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = u2f(r.v[s][k] << 16);
        x[2 * k + 1] = u2f(r.v[s][k] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = u2f(r.v[2 * s + (k >> 2)][k & 3]);
    }
    q.c[s].x = e4m3_pair<true>(x[2], x[3], e4m3_pair<false>(x[0], x[1], 0u));
    q.c[s].y = e4m3_pair<true>(x[6], x[7], e4m3_pair<false>(x[4], x[5], 0u));
  }
}

// B operand of QK: the query as bf16 (e4m3 widened exactly).
template <int FMT>
__device__ __forceinline__ void query_operands(const QueryRegs<FMT> &q, int H, int n, bf16x8 qbf[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 v;
    if constexpr (FMT == 0) {
      const uint2 x = e4m3x4_to_bf16(q.c[s].x), y = e4m3x4_to_bf16(q.c[s].y);
      v = u32x4{x.x, x.y, y.x, y.y};
    } else {
      v = q.c[s];
    }
    if (n >= H) v = u32x4{0u, 0u, 0u, 0u};
    qbf[s] = __builtin_bit_cast(bf16x8, v);
  }
}

// NVFP4: B operand of QK as f16, for the f16 MFMA (the keys widen to f16 in
// two instructions per pair, see fp4x8_to_f16_nv). Head n's 128 bf16 query
// elements (this lane: 32 of them, the other 32-element groups in lanes
// n + 16 kg) are scaled by 2^e so that the head's largest magnitude lies in
// [2^14, 2^15) (e clamped to [-113, 126] at the ends of the bf16 range):
// bf16's 8 significant bits fit f16's 11, so every element of at least 2^-28
// times the head's largest converts exactly and smaller ones to within 2^-38
// of it. The logits take inv_scale = 2^-e back (exact). Heads >= H are zero.
__device__ __forceinline__ void query_operands_f16(const QueryRegs<2> &q, int H, int n, f16x8 qh[4],
                                                   float &inv_scale) {
  uint32_t a = 0u;                                 // the head's largest |q| (fp32 bits order like values)
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int k = 0; k < 4; ++k) a = max(a, max((q.c[s][k] << 16) & 0x7FFFFFFFu, q.c[s][k] & 0x7FFF0000u));
  a = max(a, xor_lane<16>(a));
  a = max(a, xor_lane<32>(a));
  const int e = a == 0u ? 0 : min(max(141 - (int)(a >> 23), -113), 126);
  const float f = u2f((uint32_t)(127 + e) << 23);
  inv_scale = u2f((uint32_t)(127 - e) << 23);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t d = q.c[s][k];
      const f16x2 h = {(_Float16)(u2f(d << 16) * f), (_Float16)(u2f(d & 0xFFFF0000u) * f)};
      v[k] = __builtin_bit_cast(uint32_t, h);
    }
    if (n >= H) v = u32x4{0u, 0u, 0u, 0u};
    qh[s] = __builtin_bit_cast(f16x8, v);
  }
}

// The wave's token range of one selected block (page `phys`, 16 NT tokens
// from page token toff, at positions t0 ..) folded into this wave's online
// softmax state for head n = lane % 16: m_run (log2 units: the logits times
// log2 e), l_run, O. FULL: every token of the range is at or before the row's
// position (no masking); otherwise at least its first one is. FIRST: the
// wave's first range (nothing to rescale). `phys` is wave-uniform.
template <int FMT, bool FULL, bool FIRST, int NT>
__device__ __forceinline__ void attend_block(const CacheView &c, int phys, int toff, int t0, int pos,
                                             const QueryRegs<FMT> &q, int H, float qk_scale2, float &m_run,
                                             float &l_run, f32x4 O[8], int n, int kg) {
  const float NEG_INF = -__builtin_inff();
  const int64_t pb = (int64_t)phys * kPageBytes<FMT>;
  BlockRegs<FMT, NT> r;
  load_block<FMT, NT>(r, c.k_pages + pb, c.v_pages + pb, toff, n, kg);
  // The query is widened here, after the pages are requested: the empty asm
  // keeps the (loop-invariant) widening from being hoisted above these loads,
  // which would wait for the query before any page is requested.
  QueryRegs<FMT> qc = q;
#pragma unroll
  for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(qc.c[s]));
  bf16x8 qbf[4];
  f16x8 qh[4];                                    // NVFP4: the f16 query (head n scaled by 2^e)
  float q_inv = 1.0f;                             // NVFP4: 2^-e
  if constexpr (FMT == 2)
    query_operands_f16(qc, H, n, qh, q_inv);
  else
    query_operands<FMT>(qc, H, n, qbf);

  // ---- QK: scores (log2 units) of tokens 16 nt + 4 kg + i for head n
  float sc[NT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bool live = FULL || t0 + 16 * nt + n <= pos;       // the lane's A row (token 16 nt + n)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    f16x2 kb0, kb1;                                 // NVFP4: blocks 2 kg, 2 kg + 1 as f16 (1.0 = 0x38 where masked)
    if constexpr (FMT == 2) {
      const f16x2 bs = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(live ? r.kb[nt] : 0x3838u, 1.0f, false);
      kb0 = f16x2{bs.x, bs.x};
      kb1 = f16x2{bs.y, bs.y};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 a;
      if constexpr (FMT == 0) {
        uint32_t w4[4];
        fp4x8_to_bf16(live ? r.k[nt][s] : 0u, e8m0_scale(live ? r.ks[nt] : 127u), w4);
        a = u32x4{w4[0], w4[1], w4[2], w4[3]};
      } else if constexpr (FMT == 2) {
        uint32_t w4[4];
        fp4x8_to_f16_nv(live ? r.k[nt][s] : 0u, s < 2 ? kb0 : kb1, w4);
        a = u32x4{w4[0], w4[1], w4[2], w4[3]};
      } else {
        const u32x4 &src = r.k[nt][s >> 1];
        const uint2 x = e4m3x4_to_bf16(live ? src[2 * (s & 1)] : 0u);
        const uint2 y = e4m3x4_to_bf16(live ? src[2 * (s & 1) + 1] : 0u);
        a = u32x4{x.x, x.y, y.x, y.y};
      }
      if constexpr (FMT == 2)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), qh[s], acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qbf[s], acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = (FMT == 2 ? acc[i] * q_inv : acc[i]) * qk_scale2;
      if constexpr (FMT != 0) x *= r.ks[nt][i];
      sc[nt][i] = (FULL || t0 + 16 * nt + 4 * kg + i <= pos) ? x : NEG_INF;
    }
  }

  // ---- online softmax for head n (base 2)
  float bm = NEG_INF;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) bm = fmaxf(bm, sc[nt][i]);
  bm = fmaxf(bm, u2f(xor_lane<16>(f2u(bm))));
  bm = fmaxf(bm, u2f(xor_lane<32>(f2u(bm))));
  const float m_new = FIRST ? bm : fmaxf(m_run, bm);
  float ps = 0.f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[nt][i] = __builtin_amdgcn_exp2f(sc[nt][i] - m_new);      // masked tokens: 2^-inf = 0
      ps += sc[nt][i];
    }
  if constexpr (FIRST) {
    l_run = ps;
  } else {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);     // 0 when m_run is -inf
    l_run = l_run * alpha + ps;
    // rescale O rows (heads 4 kg + i) by their head's alpha
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * kg + i);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt][i] *= ai;
    }
  }
  m_run = m_new;

  // ---- PV over NT / 2 k-steps of 32 tokens
#pragma unroll
  for (int s = 0; s < NT / 2; ++s) {
    u32x4 pa;                                     // P of the lane's 8 tokens as bf16
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float p0 = sc[2 * s + (h >> 1)][2 * (h & 1)], p1 = sc[2 * s + (h >> 1)][2 * (h & 1) + 1];
      if constexpr (FMT != 0) {
        // fold V's token scale into P; masked tokens keep p = 0 (their scale may be NaN)
        const f32x4 &vs = r.vs[s][h >> 1];
        p0 = p0 == 0.0f ? 0.0f : p0 * vs[2 * (h & 1)];
        p1 = p1 == 0.0f ? 0.0f : p1 * vs[2 * (h & 1) + 1];
      }
      pa[h] = bf16_pair(p0, p1);
    }
    uint32_t W[8][4];                             // token e, byte pair cb -> bf16 pair (d = 8 n + 2 cb, + 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool live = FULL || t0 + pv_token(s, kg, e) <= pos;
      if constexpr (FMT == 0) {
        const uint32_t sb = __builtin_amdgcn_ubfe(r.vs[s][e >> 2][e & 3], 8 * (n >> 2), 8);
        fp4x8_to_bf16(live ? r.v[s][e] : 0u, e8m0_scale(live ? sb : 127u), W[e]);
      } else if constexpr (FMT == 2) {
        const uint32_t cb = __builtin_amdgcn_ubfe(r.vb[s][e], 8 * ((n >> 1) & 3), 8);   // block n / 2's code
        fp4x8_to_bf16_nv(live ? r.v[s][e] : 0u, e4m3x2_f32(live ? cb : 0x38u).x, W[e]);
      } else {
        const uint2 x = e4m3x4_to_bf16(live ? r.v[s][e].x : 0u), y = e4m3x4_to_bf16(live ? r.v[s][e].y : 0u);
        W[e][0] = x.x;
        W[e][1] = x.y;
        W[e][2] = y.x;
        W[e][3] = y.y;
      }
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const u32x4 blo = {lo_pair(W[0][cb], W[1][cb]), lo_pair(W[2][cb], W[3][cb]), lo_pair(W[4][cb], W[5][cb]),
                         lo_pair(W[6][cb], W[7][cb])};
      const u32x4 bhi = {hi_pair(W[0][cb], W[1][cb]), hi_pair(W[2][cb], W[3][cb]), hi_pair(W[4][cb], W[5][cb]),
                         hi_pair(W[6][cb], W[7][cb])};
      O[2 * cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                          __builtin_bit_cast(bf16x8, blo), O[2 * cb], 0, 0, 0);
      O[2 * cb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pa),
                                                              __builtin_bit_cast(bf16x8, bhi), O[2 * cb + 1], 0, 0, 0);
    }
  }
}

// The wave's blocks of a block list (blk_of(slot) -> block id or -1,
// phys_of(blk) -> page or -1) below slot1, folded into the wave's softmax
// state. NW waves; each block is split into 8 / NT token ranges of 16 NT
// tokens, one per wave of a group of 8 / NT consecutive waves, and wave group
// g takes slots slot0 + g, slot0 + g + NW NT / 8, ... A range that starts past
// the row's position is skipped (every range taken has a visible token). The
// first range is peeled off the loop (a loop header would make its page
// requests wait for every load still in flight, the query's included), and
// partly masked ranges take their own code path. gate(t_last) runs before a
// range's pages are requested (t_last: the range's last position).
struct NoGate {
  __device__ void operator()(int) const {}
};
template <int FMT, int NW, int NT, class BlkOf, class PhysOf, class Gate = NoGate>
__device__ __forceinline__ void attend_slots(const CacheView &c, int slot0, int slot1, int pos, const QueryRegs<FMT> &q,
                                             int H, float qk_scale2, float &m_run, float &l_run, f32x4 O[8], int n,
                                             int kg, BlkOf blk_of, PhysOf phys_of, Gate gate = Gate{}) {
  constexpr int kRanges = 8 / NT, kSpan = 16 * NT, kSlotStep = NW / kRanges;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int toff = (wave % kRanges) * kSpan;
  int slot = slot0 + wave / kRanges;
  int t0 = 0, phys = -1;
  auto next = [&]() {                            // the next slot at or after `slot` with a range to attend
    for (; slot < slot1; slot += kSlotStep) {
      const int blk = blk_of(slot);
      if (blk < 0) continue;
      t0 = blk * kTokens + toff;
      if (t0 > pos) continue;
      phys = phys_of(blk);
      if (phys >= 0) return true;
    }
    return false;
  };
  if (!next()) return;
  gate(t0 + kSpan - 1);
  if (t0 + kSpan - 1 <= pos)
    attend_block<FMT, true, true, NT>(c, phys, toff, t0, pos, q, H, qk_scale2, m_run, l_run, O, n, kg);
  else
    attend_block<FMT, false, true, NT>(c, phys, toff, t0, pos, q, H, qk_scale2, m_run, l_run, O, n, kg);
  slot += kSlotStep;
  while (next()) {
    gate(t0 + kSpan - 1);
    if (t0 + kSpan - 1 <= pos)
      attend_block<FMT, true, false, NT>(c, phys, toff, t0, pos, q, H, qk_scale2, m_run, l_run, O, n, kg);
    else
      attend_block<FMT, false, false, NT>(c, phys, toff, t0, pos, q, H, qk_scale2, m_run, l_run, O, n, kg);
    slot += kSlotStep;
  }
}

// A partial value stored device-coherent (COHERENT: an agent-scope store,
// visible to every XCD once the wave's stores are done) or plainly.
template <bool COHERENT>
__device__ __forceinline__ void put(float *p, float v) {
  if constexpr (COHERENT)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// This wave's sums for head n (m_run in log2 units) into LDS for the NW-wave
// merge: every wave leaves (m, l) and its unscaled O at once, then the one
// barrier; the merged value of each output element is then the sum over the
// waves with the factors 2^(m_w - M) (0 for a wave that saw no token).
template <int NW>
__device__ __forceinline__ void stage_waves(float (&s_m)[NW][16], float (&s_l)[NW][16],
                                            float (&s_o)[NW][16][kDim + 4], float m_run, float l_run,
                                            const f32x4 O[8]) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 15, kg = lane >> 4;
  l_run += u2f(xor_lane<16>(f2u(l_run)));
  l_run += u2f(xor_lane<32>(f2u(l_run)));
  if (kg == 0) {
    s_m[wave][n] = m_run;
    s_l[wave][n] = l_run;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 *dst = reinterpret_cast<f32x4 *>(&s_o[wave][4 * kg + i][8 * n]);
    dst[0] = f32x4{O[0][i], O[1][i], O[2][i], O[3][i]};
    dst[1] = f32x4{O[4][i], O[5][i], O[6][i], O[7][i]};
  }
  lds_barrier();
}

// Head h's merged M (log2 units), the waves' factors folded into O's 4
// elements d .. d + 3, and (LSUM) the merged l.
template <int NW, bool LSUM>
__device__ __forceinline__ f32x4 merged(const float (&s_m)[NW][16], const float (&s_l)[NW][16],
                                        const float (&s_o)[NW][16][kDim + 4], int h, int d, float &M, float &Lsum) {
  const float NEG_INF = -__builtin_inff();
  M = NEG_INF;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  Lsum = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float mw = s_m[w][h];
    const float f = (mw == NEG_INF) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
    o += *reinterpret_cast<const f32x4 *>(&s_o[w][h][d]) * f;
    if constexpr (LSUM) Lsum += (mw == NEG_INF) ? 0.0f : s_l[w][h] * f;
  }
  return o;
}

// The workgroup's partial (m, l, O) of partition p from the staged waves; m is
// stored in natural-log units.
template <bool COHERENT, int NW>
__device__ __forceinline__ void write_partial(float (&s_m)[NW][16], float (&s_l)[NW][16],
                                              float (&s_o)[NW][16][kDim + 4], float m_run, float l_run,
                                              const f32x4 O[8], int row, int H, int P, int p, int mls,
                                              float *__restrict__ sp_m,
                                              float *__restrict__ sp_l, float *__restrict__ sp_o) {
  const float NEG_INF = -__builtin_inff();
  stage_waves<NW>(s_m, s_l, s_o, m_run, l_run, O);
  const int64_t part = (int64_t)row * H;      // + h, then * P + p
  float *const row_o = sp_o + part * P * kDim;
  const __amdgpu_buffer_rsrc_t ro = row_rsrc(row_o, H * P * kDim);
#pragma unroll
  for (int rr = 0; rr < 512 / (64 * NW); ++rr) {   // 16 heads x 32 float4 of O
    const int idx = threadIdx.x + 64 * NW * rr;
    const int h = idx >> 5, d = 4 * (idx & 31);
    if (h < H) {
      float M, unused;
      const f32x4 o = merged<NW, false>(s_m, s_l, s_o, h, d, M, unused);
      const int32_t off = (h * P + p) * kDim + d;
      if constexpr (COHERENT)
        store4_coherent(ro, off, o);
      else
        *reinterpret_cast<f32x4 *>(row_o + off) = o;
    }
  }
  if (threadIdx.x < (unsigned)H) {
    const int h = threadIdx.x;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      Lsum += (s_m[w][h] == NEG_INF) ? 0.0f : s_l[w][h] * __builtin_amdgcn_exp2f(s_m[w][h] - M);
    put<COHERENT>(sp_m + (int64_t)row * mls + h * P + p, M * kLn2);
    put<COHERENT>(sp_l + (int64_t)row * mls + h * P + p, Lsum);
  }
}

// A row attended by one partition: the staged waves merged straight into the
// row's output (O / l as bf16, lse = m + ln l), the same values the merge of a
// single partition gives (its weight is exactly 1).
template <int NW>
__device__ __forceinline__ void write_row(float (&s_m)[NW][16], float (&s_l)[NW][16], float (&s_o)[NW][16][kDim + 4],
                                          float m_run, float l_run, const f32x4 O[8], int row, int H,
                                          uint16_t *__restrict__ out, float *__restrict__ lse) {
  stage_waves<NW>(s_m, s_l, s_o, m_run, l_run, O);
#pragma unroll
  for (int rr = 0; rr < 512 / (64 * NW); ++rr) {   // 16 heads x 32 groups of 4 elements
    const int idx = threadIdx.x + 64 * NW * rr;
    const int h = idx >> 5, d = 4 * (idx & 31);
    if (h < H) {
      float M, Lsum;
      const f32x4 o = merged<NW, true>(s_m, s_l, s_o, h, d, M, Lsum);
      const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
      const int64_t r = (int64_t)row * H + h;
      uint2 packed;
      packed.x = bf16_pair(o[0] * inv, o[1] * inv);
      packed.y = bf16_pair(o[2] * inv, o[3] * inv);
      uint16_t *const dst = out + r * kDim + d;                      // out: at least 4-byte aligned
      if ((reinterpret_cast<uintptr_t>(out) & 7) == 0) {
        *reinterpret_cast<uint2 *>(dst) = packed;
      } else {
        reinterpret_cast<uint32_t *>(dst)[0] = packed.x;
        reinterpret_cast<uint32_t *>(dst)[1] = packed.y;
      }
      // an explicit fma: the same rounding in every kernel this is inlined into
      if (lse && d == 0) lse[r] = Lsum > 0.0f ? __builtin_fmaf(M, kLn2, __logf(Lsum)) : -__builtin_inff();
    }
  }
}

template <int FMT, int TILES>
__global__ __launch_bounds__(256) void k_split_attn(CacheView c, const void *__restrict__ qv,
                                                    const int32_t *__restrict__ block_table,
                                                    int32_t q_rows, int32_t H, int32_t topk, int32_t P,
                                                    float sm_scale, float *__restrict__ sp_m,
                                                    float *__restrict__ sp_l, float *__restrict__ sp_o) {
  __shared__ float s_m[kAttnWaves][16], s_l[kAttnWaves][16];
  __shared__ float s_o[kAttnWaves][16][kDim + 4];
  const int p = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int row = b * q_rows + j;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int pos = c.context_lens[b] - q_rows + j;
  const int cps = (topk + P - 1) / P;
  const int slot0 = p * cps, slot1 = min(slot0 + cps, (int)topk);
  QueryRegs<FMT> qr;
  load_query<FMT>(qv, row, H, n, kg, qr);

  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  attend_slots<FMT, kAttnWaves, TILES>(
      c, slot0, slot1, pos, qr, H, sm_scale * kLog2e, m_run, l_run, O, n, kg,
      [&](int slot) {
        const int blk = __builtin_amdgcn_readfirstlane(block_table[(int64_t)row * topk + slot]);
        return (blk < 0 || blk >= c.stride || blk * kTokens > pos) ? -1 : blk;
      },
      [&](int blk) {
        const int phys = __builtin_amdgcn_readfirstlane(c.page_table[(int64_t)b * c.stride + blk]);
        return (phys < 0 || phys >= c.num_pages) ? -1 : phys;
      });
  write_partial<false, kAttnWaves>(s_m, s_l, s_o, m_run, l_run, O, row, H, P, p, H * P, sp_m, sp_l, sp_o);
}

// Shared memory of one decode-step attention workgroup.
template <int ITEMS, bool SELECT>
struct StepAttnSmem {
  TopkSmem<SELECT ? ITEMS : 1, kStepWaves> tk;
  int32_t s_pt[64 * kStepWaves * ITEMS];
  float s_m[kStepWaves][16], s_l[kStepWaves][16];
  float s_o[kStepWaves][16][kDim + 4];
  uint32_t s_last, s_local;                        // merging workgroup; all arrivals on its XCC
};

// What the attention workgroups of the single-launch decode step wait for:
// the scoring workgroups of their sequence (seq_cnt[2 b] counts them in, up
// to n_score each) — and once every attention workgroup of the sequence has
// passed (seq_cnt[2 b + 1] counts them), the last one sets both words back to
// zero for the next launch. Null in the two-launch step.
struct StepWait {
  uint32_t *seq_cnt = nullptr;     // [B][2]
  uint32_t n_score = 0;            // scoring workgroups per sequence
};

// Spin limit of the wait (iterations of ~128 clocks each, about a quarter of
// a second): a bound that every wave reaches even if a count never arrives.
constexpr uint32_t kWaitSpins = 1u << 21;

// How an attention workgroup gets what other workgroups of the same launch
// wrote. kTwoLaunch: nothing (the scores and e4m3 query come from an earlier
// launch). kOneLaunchStep: the single-launch decode step — wait for the
// sequence's scoring workgroups first, then read the scores and the e4m3 query
// device-coherently. kOneLaunchReuse: the single-launch reuse step — the query
// is rounded to e4m3 in registers from the caller's fp32 / bf16 query (MXFP4
// K / V), and only a wave whose token range holds the step's new positions
// waits, just before requesting those pages, for the sequence's store
// workgroups.
enum AttnMode { kTwoLaunch = 0, kOneLaunchStep = 1, kOneLaunchReuse = 2 };

// The single-launch reuse step's bookkeeping of sequence b, run by the
// workgroup that completes one of the sequence's rows (its merging workgroup,
// or the only one when P = 1): the last of the q_rows takes the store count
// seq_cnt[2 b] back by q_rows (a subtraction, so that a store workgroup's
// count arriving after it still nets to zero when the launch ends) and clears
// its own counter seq_cnt[2 b + 1]. Every wait of the sequence precedes its
// workgroup's arrival and so precedes this.
__device__ __forceinline__ void reuse_row_done(const StepWait &sw, int b, int q_rows) {
  if (__hip_atomic_fetch_add(sw.seq_cnt + 2 * b + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
      (uint32_t)(q_rows - 1)) {
    __hip_atomic_fetch_sub(sw.seq_cnt + 2 * b, (uint32_t)q_rows, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(sw.seq_cnt + 2 * b + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The decode step's attention workgroup (partition p of query row j of
// sequence b). SELECT: the workgroup first selects its row's top-k blocks
// itself (the workgroup selection of topk.hpp over the row's scores) and
// partition 0 writes the row's block table; otherwise the row's blocks come
// from a given block table (a selection reused from an earlier layer;
// entries < 0, past the table or past the row's position are skipped). The
// row's page table is staged in LDS. Everything the workgroup needs from
// memory before the K / V pages — the context length, the score row or table
// row and the page-table row — is requested in one round trip; the query goes
// out with the first block's pages. MODE: see AttnMode. (In the single-launch
// modes the K / V pages holding the step's new rows are read only after the
// wait for their stores, so no stale copy of them can be in this XCD's L2: it
// holds no line that was not fetched in this launch, and every wave that
// reads those pages has waited first.) q_dtype: the caller's query dtype
// (kOneLaunchReuse with MXFP4 K / V only).
template <int FMT, int ITEMS, bool SELECT, int MODE, int TILES>
__device__ __forceinline__ void step_attn_wg(const CacheView &c, const float *__restrict__ scores,
                                             const void *__restrict__ qv, int32_t q_rows, int32_t H, int32_t topk,
                                             int32_t P, float sm_scale, int32_t *__restrict__ block_table,
                                             float *__restrict__ sp_m, float *__restrict__ sp_l,
                                             float *__restrict__ sp_o, const FusedMerge &fm, const StepWait &sw,
                                             int p, int j, int b, StepAttnSmem<ITEMS, SELECT> &sm, int q_dtype = 0) {
  constexpr int NT = 64 * kStepWaves;              // threads
  constexpr bool RAWQ = MODE == kOneLaunchReuse && FMT == 0;
  static_assert(MODE != kOneLaunchReuse || !SELECT, "the reuse step selects nothing");
  const int row = b * q_rows + j;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 15, kg = lane >> 4;
  const int stride = c.stride;

  const int L = c.context_lens[b];
  float v[ITEMS];
  int32_t pt[ITEMS];
  int32_t given = -1;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r) {
    const int i = min(tid + NT * r, stride - 1);   // clamped: unconditional loads
    if constexpr (SELECT && MODE == kTwoLaunch) v[r] = scores[(int64_t)row * stride + i];
    pt[r] = c.page_table[(int64_t)b * stride + i];
  }
  if constexpr (!SELECT) given = block_table[(int64_t)row * topk + min(lane, topk - 1)];
  RawQuery raw;
  if constexpr (RAWQ) load_query_raw(qv, q_dtype, row, H, n, kg, raw);
  if constexpr (MODE == kOneLaunchStep) {
    // the sequence's scores, new K / V rows and e4m3 query are complete once
    // all its scoring workgroups have counted in
    if (tid == 0) {
      uint32_t spins = 0;
      while (__hip_atomic_load(sw.seq_cnt + 2 * b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < sw.n_score &&
             ++spins < kWaitSpins)
        __builtin_amdgcn_s_sleep(2);
      // every attention workgroup of the sequence past the wait: reset both words
      if (__hip_atomic_fetch_add(sw.seq_cnt + 2 * b + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
          (uint32_t)(q_rows * P - 1)) {
        __hip_atomic_store(sw.seq_cnt + 2 * b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(sw.seq_cnt + 2 * b + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if constexpr (SELECT) {
#pragma unroll
      for (int r = 0; r < ITEMS; ++r) {
        const int i = min(tid + NT * r, stride - 1);
        v[r] = __hip_atomic_load(scores + (int64_t)row * stride + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  const int pos = L - q_rows + j;
#pragma unroll
  for (int r = 0; r < ITEMS; ++r)
    if (tid + NT * r < stride) sm.s_pt[tid + NT * r] = pt[r];
  int n_sel;
  uint32_t sel;
  if constexpr (SELECT) {
    const int n_cand = pos < 0 ? 0 : min(pos / kTokens + 1, stride);
    sel = wg_topk<ITEMS, kStepWaves>(v, n_cand, topk, sm.tk, n_sel);
    lds_barrier();                                 // s_pt (the selection may return before any barrier)
    if (p == 0 && tid < topk) block_table[(int64_t)row * topk + tid] = tid < n_sel ? (int32_t)sel : -1;
  } else {
    sel = (uint32_t)given;                         // lane s: slot s (lanes >= topk are never read)
    n_sel = topk;
    lds_barrier();                                 // s_pt
  }

  const int cps = (topk + P - 1) / P;
  const int slot0 = p * cps, slot1 = min(slot0 + cps, n_sel);
  QueryRegs<FMT> qr;                               // widened after the first block's pages are requested
  if constexpr (RAWQ)
    round_query_e4m3(raw, q_dtype, qr);
  else
    load_query<FMT, MODE == kOneLaunchStep && FMT == 0>(qv, row, H, n, kg, qr);   // e4m3 written in the same launch
  float m_run = -__builtin_inff(), l_run = 0.0f;
  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto blk_of = [&](int slot) {
    const int blk = __builtin_amdgcn_readlane((int)sel, slot);
    if constexpr (SELECT) return blk;              // a candidate: 0 <= blk, blk * 128 <= pos
    return (blk < 0 || blk >= stride || blk * kTokens > pos) ? -1 : blk;
  };
  auto phys_of = [&](int blk) {
    const int phys = __builtin_amdgcn_readfirstlane(sm.s_pt[blk]);
    return (phys < 0 || phys >= c.num_pages) ? -1 : phys;
  };
  if constexpr (MODE == kOneLaunchReuse) {
    // a range reaching the step's new positions (L - q_rows ..) waits for the
    // sequence's store workgroups (bounded)
    const int new0 = L - q_rows;
    attend_slots<FMT, kStepWaves, TILES>(
        c, slot0, slot1, pos, qr, H, sm_scale * kLog2e, m_run, l_run, O, n, kg, blk_of, phys_of, [&](int t_last) {
          if (t_last < new0) return;
          uint32_t spins = 0;
          while ((uint32_t)__builtin_amdgcn_readfirstlane((int)__hip_atomic_load(
                     sw.seq_cnt + 2 * b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) < sw.n_score &&
                 ++spins < kWaitSpins)
            __builtin_amdgcn_s_sleep(2);
        });
  } else {
    attend_slots<FMT, kStepWaves, TILES>(c, slot0, slot1, pos, qr, H, sm_scale * kLog2e, m_run, l_run, O, n, kg,
                                              blk_of, phys_of);
  }
  if (P == 1) {                                     // the row is this workgroup's alone: no exchange
    write_row<kStepWaves>(sm.s_m, sm.s_l, sm.s_o, m_run, l_run, O, row, H, fm.out, fm.lse);
    if constexpr (MODE == kOneLaunchReuse)
      if (tid == 0) reuse_row_done(sw, b, q_rows);
    return;
  }
  const int mls = step_ml_stride(H, P);
  write_partial<true, kStepWaves>(sm.s_m, sm.s_l, sm.s_o, m_run, l_run, O, row, H, P, p, mls, sp_m, sp_l, sp_o);

  // ---- the row's merge, by its last partition workgroup to finish. The
  // partials went out as agent-scope (device-coherent) stores; once every
  // wave's stores are done (vmcnt) and the workgroup has met, one arrival is
  // counted (device-scope atomic): 1 in bits 0-7 and 1 in the 7-bit field of
  // the workgroup's XCC (bits 8 + 7 x; P <= 64 keeps both from overflowing).
  // The workgroup that takes the count to P reads every partition's partials:
  // through its XCD's L2 when all P arrivals came from its own XCC (the
  // placement of xcd_item makes that the usual case), with agent-scope loads
  // otherwise. Plain loads are safe then: the partials reached that L2 (or
  // memory) before their arrivals were counted, and this CU's L1 holds no
  // line of them (L1 starts empty in a launch, only a row's merger reads its
  // partials, and rows do not share lines: step_ml_stride). No cache
  // write-back or invalidate is needed on either side.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if (tid == 0) {
    const uint32_t x = xcc_id();
    const uint64_t inc = 1ull + (1ull << (8 + 7 * x));
    const uint64_t old = __hip_atomic_fetch_add(fm.counters + row, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.s_last = (uint32_t)(old & 0xFFu) == (uint32_t)(P - 1);
    sm.s_local = (uint32_t)(((old + inc) >> (8 + 7 * x)) & 0x7Fu) == (uint32_t)P;
  }
  lds_barrier();
  if (!sm.s_last) return;
  if (tid == 0) {
    fm.counters[row] = 0ull;                      // every arrival is in: the row's counter is free for the next launch
    if constexpr (MODE == kOneLaunchReuse) reuse_row_done(sw, b, q_rows);
  }
  if (sm.s_local)
    merge_row<false>(sp_m, sp_l, sp_o, row, H, P, mls, fm.out, fm.lse);
  else
    merge_row<true>(sp_m, sp_l, sp_o, row, H, P, mls, fm.out, fm.lse);
}

// Work item of attention workgroup `lin` of a grid of n: workgroups are
// dispatched to the 8 XCDs round robin by id (XCD = id % 8, checked on
// MI355X with the hardware XCC id register), so when n is a multiple of 8
// the items are dealt so that each XCD takes a run of consecutive items: a
// row's partitions, and the rows of one sequence, share one XCD and its L2
// (the score and page-table rows, the K / V pages the rows have in common).
// Results do not depend on it.
__device__ __forceinline__ int xcd_item(int lin, int n) {
  return (n & 7) == 0 ? (lin & 7) * (n >> 3) + (lin >> 3) : lin;
}

template <int FMT, int ITEMS, bool SELECT, int TILES>
__global__ __launch_bounds__(64 * kStepWaves) void k_select_attn(CacheView c, const float *__restrict__ scores,
                                                     const void *__restrict__ qv, int32_t q_rows, int32_t H,
                                                     int32_t topk, int32_t P, float sm_scale,
                                                     int32_t *__restrict__ block_table, float *__restrict__ sp_m,
                                                     float *__restrict__ sp_l, float *__restrict__ sp_o,
                                                     FusedMerge fm) {
  __shared__ StepAttnSmem<ITEMS, SELECT> sm;
  const int r = xcd_item(blockIdx.x, gridDim.x);   // item r: partition r % P, row (r / P) % q_rows, sequence
  step_attn_wg<FMT, ITEMS, SELECT, kTwoLaunch, TILES>(c, scores, qv, q_rows, H, topk, P, sm_scale, block_table, sp_m,
                                                      sp_l, sp_o, fm, StepWait{}, r % P, (r / P) % q_rows,
                                                      r / (P * q_rows), sm);
}

// ---------------------------------------------------------------- the step as one launch
// The whole decode step in one grid: the scoring workgroups first (ids below
// B ny: sequence id % B, wave group id / B, the two-launch scorer's 4-wave x
// 8-page x 3-stage shape), then the attention workgroups (partition, row,
// sequence). A scoring workgroup writes its scores, its share of the step's
// K / V rows and of the e4m3 query with device-coherent stores, waits for
// them to complete and counts itself in for its sequence. An attention
// workgroup loads its context length and page-table row, waits for its
// sequence's count, then selects, attends and merges as in the two-launch
// step. Workgroups are dispatched in increasing id order on each XCD, so an
// attention workgroup only ever waits for scoring workgroups that were
// dispatched before it, and those wait for nothing: the wait always ends, and
// it is also bounded (kWaitSpins). Attention workgroups of a sequence start
// as soon as the CUs that scored free up, so their launch and prologue
// overlap the rest of the scan instead of following it.
template <int MT, int ITEMS>
constexpr int kStepLds = kScoreLds<MT, 0, 4, 3> > (int)sizeof(StepAttnSmem<ITEMS, true>)
                             ? kScoreLds<MT, 0, 4, 3>
                             : (int)sizeof(StepAttnSmem<ITEMS, true>);

template <int MT, int ITEMS, int TILES>
__global__ __launch_bounds__(64 * kStepWaves) void k_decode_step(
    CacheView c, const uint16_t *__restrict__ q_idx, const float *__restrict__ w, int32_t q, int32_t H_I,
    float *__restrict__ scores, StepStore st, int32_t B, int32_t ny, int32_t H, int32_t topk, int32_t P,
    float sm_scale, int32_t *__restrict__ block_table, float *__restrict__ sp_m, float *__restrict__ sp_l,
    float *__restrict__ sp_o, FusedMerge fm, StepWait sw) {
  // one LDS object, used by either role
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStepLds<MT, ITEMS>];
  const int n_score = B * ny;
  if ((int)blockIdx.x < n_score) {
    const int b = (int)blockIdx.x % B, gy = (int)blockIdx.x / B;
    index_score_wg<MT, 0, 4, 8, 3, true>(c, q_idx, w, q, H_I, scores, st, b, gy, ny, lds);
    // every store of this workgroup done (vmcnt counts stores too), then one
    // arrival for the sequence
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(sw.seq_cnt + 2 * b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int a = xcd_item((int)blockIdx.x - n_score, (int)gridDim.x - n_score);   // XCD runs when 8 divides n_score
  const int p = a % P, j = (a / P) % q, b = a / (P * q);
  step_attn_wg<0, ITEMS, true, kOneLaunchStep, TILES>(c, scores, st.q8, q, H, topk, P, sm_scale, block_table, sp_m,
                                                      sp_l, sp_o, fm, sw, p, j, b,
                                                      *reinterpret_cast<StepAttnSmem<ITEMS, true> *>(lds));
}

// ---------------------------------------------------------------- the reuse step as one launch
// The step of a layer that reuses a block selection in one grid: one store
// workgroup per query row first (ids below B q_rows: the row's new K and V
// rows, device-coherent; then it counts itself in for its sequence), then the
// attention workgroups (partition, row, sequence) over the given table
// (kOneLaunchReuse: the query rounded to e4m3 in registers for MXFP4 K / V;
// only the ranges that hold the step's new positions wait for the sequence's
// store workgroups). The store workgroups wait for nothing and are
// dispatched first (increasing ids per XCD), so every wait ends; it is also
// bounded (kWaitSpins). The merge counters and the sequence counters
// (seq_cnt) must be zero before the first launch and are left zero.
template <int FMT, int ITEMS, int TILES>
__global__ __launch_bounds__(64 * kStepWaves) void k_reuse_step(
    CacheView c, const float *__restrict__ k_new, const float *__restrict__ v_new, const void *__restrict__ q_src,
    int32_t q_dtype, int32_t q_rows, int32_t H, int32_t topk, int32_t P, float sm_scale,
    const int32_t *__restrict__ block_table, float *__restrict__ sp_m, float *__restrict__ sp_l,
    float *__restrict__ sp_o, FusedMerge fm, StepWait sw, int32_t n_store) {
  __shared__ StepAttnSmem<ITEMS, false> sm;
  if ((int)blockIdx.x < n_store) {
    const int row = blockIdx.x;
    reuse_store_wg<true>(c, k_new, v_new, nullptr, 0, H, nullptr, nullptr, q_rows, row);
    // every store of this workgroup done, then one arrival for the sequence
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(sw.seq_cnt + 2 * (row / q_rows), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int a = xcd_item((int)blockIdx.x - n_store, (int)gridDim.x - n_store);
  const int p = a % P, j = (a / P) % q_rows, b = a / (P * q_rows);
  step_attn_wg<FMT, ITEMS, false, kOneLaunchReuse, TILES>(c, nullptr, q_src, q_rows, H, topk, P, sm_scale,
                                                          const_cast<int32_t *>(block_table), sp_m, sp_l, sp_o, fm,
                                                          sw, p, j, b, sm, q_dtype);
}

hipError_t launch_reuse_step(const CacheView &c, const float *k_new, const float *v_new, const void *q, int q_dtype,
                             const int32_t *block_table, int32_t B, int32_t q_rows, int32_t H, int32_t topk,
                             int32_t P, float sm_scale, float *sp_m, float *sp_l, float *sp_o, const FusedMerge &fm,
                             uint32_t *seq_cnt, hipStream_t s) {
  if (B * q_rows == 0) return hipSuccess;
  constexpr int NT = 64 * kStepWaves;
  StepWait sw;
  sw.seq_cnt = seq_cnt;
  sw.n_score = (uint32_t)q_rows;                   // store workgroups per sequence
  const int n_store = B * q_rows;
  const dim3 grid((unsigned)(n_store + B * q_rows * P)), block(NT);
#define MXS_REUSE_T(F, I, T)                                                                                     \
  hipLaunchKernelGGL((k_reuse_step<F, I, T>), grid, block, 0, s, c, k_new, v_new, q, q_dtype, q_rows, H, topk, P, \
                     sm_scale, block_table, sp_m, sp_l, sp_o, fm, sw, n_store)
#define MXS_REUSE(F, I)                                            \
  do {                                                             \
    if (step_tiles(topk, P) == 4) MXS_REUSE_T(F, I, 4);            \
    else MXS_REUSE_T(F, I, 8);                                     \
  } while (0)
#define MXS_REUSE_FMT(F)                            \
  if (c.stride <= NT * 2) MXS_REUSE(F, 2);          \
  else if (c.stride <= NT * 8) MXS_REUSE(F, 8);     \
  else MXS_REUSE(F, 32)
  if (c.kv_format == 0) {
    MXS_REUSE_FMT(0);
  } else if (c.kv_format == 1) {
    MXS_REUSE_FMT(1);
  } else {
    MXS_REUSE_FMT(2);
  }
#undef MXS_REUSE_FMT
#undef MXS_REUSE
#undef MXS_REUSE_T
  return hipGetLastError();
}

bool decode_step_one_launch(const CacheView &c, int32_t B, int32_t q) {
  return c.kv_format == 0 && c.idx_format == 0 && q <= 8 && (int64_t)B * c.stride >= 256 * 32;
}

template <int MT>
static void launch_step_mt(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                           int32_t H_I, float *scores, const StepStore &st, int32_t H, int32_t topk, int32_t P,
                           float sm_scale, int32_t *block_table, float *sp_m, float *sp_l, float *sp_o,
                           const FusedMerge &fm, uint32_t *seq_cnt, hipStream_t s) {
  constexpr int NT = 64 * kStepWaves;
  const int ny = (c.stride + 32 - 1) / 32;         // 4 waves x 8 pages per scoring workgroup
  StepWait sw;
  sw.seq_cnt = seq_cnt;
  sw.n_score = (uint32_t)ny;
  const dim3 grid((unsigned)(B * ny + B * q * P)), block(NT);
#define MXS_STEP_T(I, T)                                                                                         \
  hipLaunchKernelGGL((k_decode_step<MT, I, T>), grid, block, 0, s, c, q_idx, w, q, H_I, scores, st, B, ny, H,      \
                     topk, P, sm_scale, block_table, sp_m, sp_l, sp_o, fm, sw)
#define MXS_STEP(I)                                                \
  do {                                                             \
    if (step_tiles(topk, P) == 4) MXS_STEP_T(I, 4);                \
    else MXS_STEP_T(I, 8);                                         \
  } while (0)
  if (c.stride <= NT * 2) MXS_STEP(2);
  else if (c.stride <= NT * 8) MXS_STEP(8);
  else MXS_STEP(32);
#undef MXS_STEP
#undef MXS_STEP_T
}

hipError_t launch_decode_step(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                              int32_t H_I, float *scores, const StepStore &st, int32_t H, int32_t topk, int32_t P,
                              float sm_scale, int32_t *block_table, float *sp_m, float *sp_l, float *sp_o,
                              const FusedMerge &fm, uint32_t *seq_cnt, hipStream_t s) {
  if (B * q == 0) return hipSuccess;
  if (q <= 4)
    launch_step_mt<1>(c, q_idx, w, B, q, H_I, scores, st, H, topk, P, sm_scale, block_table, sp_m, sp_l, sp_o, fm,
                      seq_cnt, s);
  else
    launch_step_mt<2>(c, q_idx, w, B, q, H_I, scores, st, H, topk, P, sm_scale, block_table, sp_m, sp_l, sp_o, fm,
                      seq_cnt, s);
  return hipGetLastError();
}

hipError_t launch_split_attn(const CacheView &c, const void *q, int q_dtype, const int32_t *block_table,
                             int32_t B, int32_t q_rows, int32_t H, int32_t topk, int32_t P, float sm_scale,
                             float *sp_m, float *sp_l, float *sp_o, hipStream_t s) {
  (void)q_dtype;
  if (B * q_rows == 0) return hipSuccess;
  const dim3 grid((unsigned)P, (unsigned)q_rows, (unsigned)B);
#define MXS_SPLIT(F, T)                                                                                     \
  hipLaunchKernelGGL((k_split_attn<F, T>), grid, dim3(256), 0, s, c, q, block_table, q_rows, H, topk, P,   \
                     sm_scale, sp_m, sp_l, sp_o)
  const bool half = step_tiles(topk, P) == 4;
  if (c.kv_format == 0) {
    if (half) MXS_SPLIT(0, 4); else MXS_SPLIT(0, 8);
  } else if (c.kv_format == 1) {
    if (half) MXS_SPLIT(1, 4); else MXS_SPLIT(1, 8);
  } else {
    if (half) MXS_SPLIT(2, 4); else MXS_SPLIT(2, 8);
  }
#undef MXS_SPLIT
  return hipGetLastError();
}

template <bool SELECT>
static void launch_attn_items(const CacheView &c, const float *scores, const void *q, int32_t B, int32_t q_rows,
                              int32_t H, int32_t topk, int32_t P, float sm_scale, int32_t *block_table, float *sp_m,
                              float *sp_l, float *sp_o, const FusedMerge &fm, hipStream_t s) {
  constexpr int NT = 64 * kStepWaves;
  const dim3 grid((unsigned)(P * q_rows * B)), block(NT);
#define MXS_SELECT_ATTN_T(F, I, T)                                                                               \
  hipLaunchKernelGGL((k_select_attn<F, I, SELECT, T>), grid, block, 0, s, c, scores, q, q_rows, H, topk, P,     \
                     sm_scale, block_table, sp_m, sp_l, sp_o, fm)
#define MXS_SELECT_ATTN(F, I)                                      \
  do {                                                             \
    if (step_tiles(topk, P) == 4) MXS_SELECT_ATTN_T(F, I, 4);      \
    else MXS_SELECT_ATTN_T(F, I, 8);                               \
  } while (0)
  static_assert(NT * 32 >= MXS_MAX_PAGES_PER_SEQ, "candidates per thread");
  if (c.kv_format == 0) {
    if (c.stride <= NT * 2) MXS_SELECT_ATTN(0, 2);
    else if (c.stride <= NT * 8) MXS_SELECT_ATTN(0, 8);
    else MXS_SELECT_ATTN(0, 32);
  } else if (c.kv_format == 1) {
    if (c.stride <= NT * 2) MXS_SELECT_ATTN(1, 2);
    else if (c.stride <= NT * 8) MXS_SELECT_ATTN(1, 8);
    else MXS_SELECT_ATTN(1, 32);
  } else {
    if (c.stride <= NT * 2) MXS_SELECT_ATTN(2, 2);
    else if (c.stride <= NT * 8) MXS_SELECT_ATTN(2, 8);
    else MXS_SELECT_ATTN(2, 32);
  }
#undef MXS_SELECT_ATTN
#undef MXS_SELECT_ATTN_T
}

hipError_t launch_select_attn(const CacheView &c, const float *scores, const void *q, int32_t B, int32_t q_rows,
                              int32_t H, int32_t topk, int32_t P, float sm_scale, int32_t *block_table, float *sp_m,
                              float *sp_l, float *sp_o, const FusedMerge &fm, hipStream_t s) {
  if (B * q_rows == 0) return hipSuccess;
  launch_attn_items<true>(c, scores, q, B, q_rows, H, topk, P, sm_scale, block_table, sp_m, sp_l, sp_o, fm, s);
  return hipGetLastError();
}

hipError_t launch_table_attn(const CacheView &c, const int32_t *block_table, const void *q, int32_t B, int32_t q_rows,
                             int32_t H, int32_t topk, int32_t P, float sm_scale, float *sp_m, float *sp_l, float *sp_o,
                             const FusedMerge &fm, hipStream_t s) {
  if (B * q_rows == 0) return hipSuccess;
  launch_attn_items<false>(c, nullptr, q, B, q_rows, H, topk, P, sm_scale, const_cast<int32_t *>(block_table), sp_m,
                           sp_l, sp_o, fm, s);
  return hipGetLastError();
}

}  // namespace mxs
