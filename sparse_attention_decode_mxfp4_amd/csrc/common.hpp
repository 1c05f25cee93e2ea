// Device-side helpers shared by the mxsparse kernels (gfx950, wave64).
//
// Number formats (OCP Microscaling Formats v1.0 for e2m1 / e8m0, OCP FP8 for
// e4m3; the pages name the formats, ATOM PR #2812 "Mono decode over the MXFP4
// KV and index caches", commit messages; NVFP4 is named in ATOM PR #2686,
// timeline entry #2744, and read as e2m1 in 16-element blocks with e4m3 block
// scales and a per-token fp32 scale):
//   e2m1  1 sign, 2 exponent, 1 mantissa bit: +-{0, .5, 1, 1.5, 2, 3, 4, 6}
//   e8m0  a power of two 2^(byte - 127); byte 255 is NaN
//   e4m3  bias 7, max 448, 0x7F / 0xFF NaN, subnormals m * 2^-9
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxs {

constexpr int kTokens = 128;           // tokens per page (= one block)
constexpr int kDim = 128;              // head_dim
constexpr int kMxPageBytes = 8704;     // 128 * 64 data + 128 * 4 scale bytes
constexpr int kMxScaleOff = 8192;
constexpr int kF8PageBytes = 16896;    // 128 * 128 codes + 128 fp32 scales
constexpr int kF8ScaleOff = 16384;
constexpr int kNvPageBytes = 9728;     // 128 * 64 codes + 128 * 8 e4m3 block scales + 128 fp32 token scales
constexpr int kNvBScaleOff = 8192;
constexpr int kNvTScaleOff = 9216;

// Page bytes of a cache format (0 MXFP4, 1 FP8, 2 NVFP4).
template <int FMT>
constexpr int kPageBytes = FMT == 0 ? kMxPageBytes : (FMT == 1 ? kF8PageBytes : kNvPageBytes);

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ---------------------------------------------------------------- MXFP4 encode
// e8m0 byte of a 32-element group from the fp32 bits of its largest magnitude:
// OCP MX scale 2^(floor(log2 amax) - 2); floor(log2 amax) is the unbiased
// exponent E - 127 of a normal amax, so the byte is E - 2, clamped at 0 (zero
// and subnormal groups take the smallest scale).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 23;
  return e > 2u ? e - 2u : 0u;
}

// 2^(127 - byte): multiplying by it divides by the group scale exactly
// (byte <= 252 for finite input, so the factor stays a normal fp32).
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) { return u2f((254u - byte) << 23); }

// e2m1 code of an already scaled value: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6},
// ties to the even code (0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4), magnitudes above 6 saturate; sign bit 3 from the input.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = __builtin_fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((f2u(v) >> 28) & 8u);
}

// ---------------------------------------------------------------- e4m3 encode
// Saturating OCP e4m3 code: round to nearest even, |x| >= 448 and inf -> 448,
// NaN -> 0x7F, sign bit kept.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = f2u(x);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return s | 0x7Fu;            // NaN
  if (a >= 0x43E00000u) return s | 0x7Eu;           // >= 448, inf
  if (a < 0x3C800000u) {                            // below 2^-6: grid m * 2^-9, m = 0..8
    const float t = u2f(a) * 512.0f;                // exact scaling
    return s | (uint32_t)__builtin_rintf(t);        // rint: round half to even
  }
  // normal: keep 3 mantissa bits, round half to even, rebias 127 -> 7
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  return s | (r - (120u << 3));
}

// ---------------------------------------------------------------- decode to bf16
// fp32 value of the e8m0 scale byte, as the cvt_scalef32 instructions take it.
__device__ __forceinline__ float e8m0_f32(uint32_t byte) {
  return byte ? u2f(byte << 23) : u2f(0x00400000u);   // byte 0 is 2^-127 (an fp32 subnormal)
}

// Two e2m1 codes (byte `sel` of `packed`: low nibble first) times 2^(byte-127)
// as two bf16 values; exact for every scale that keeps the result normal.
#define MXS_CVT_FP4_BF16(packed, scale_f32, sel) \
  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((packed), (scale_f32), (sel))

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// The four bytes of `packed` (8 e2m1 codes) as four bf16 pairs, scaled.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t packed, float scale_f32, uint32_t out[4]) {
  out[0] = bf16x2_bits(MXS_CVT_FP4_BF16(packed, scale_f32, 0));
  out[1] = bf16x2_bits(MXS_CVT_FP4_BF16(packed, scale_f32, 1));
  out[2] = bf16x2_bits(MXS_CVT_FP4_BF16(packed, scale_f32, 2));
  out[3] = bf16x2_bits(MXS_CVT_FP4_BF16(packed, scale_f32, 3));
}

// Two fp32 as a bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The e4m3 codes in bytes 0 and 1 of `d` as fp32 (exact; 0x7F / 0xFF give NaN).
__device__ __forceinline__ float2 e4m3x2_f32(uint32_t d) {
  const uint32_t b = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false));
  return make_float2(u2f(b << 16), u2f(b & 0xFFFF0000u));
}

// NVFP4 widening: the eight e2m1 codes of `packed` (low nibble first) times an
// e4m3 block scale `sc` (given as its exact fp32 value) as four bf16 pairs.
// The scaled convert instructions apply only a power of two, so the codes are
// widened unscaled to fp32 and multiplied there: an e2m1 value has at most 2
// significant bits and an e4m3 value at most 4, so the product (<= 6 bits,
// between 2^-10 and 2688) is exact in fp32 and again in bf16.
#define MXS_NV_PAIR(k)                                                       \
  do {                                                                       \
    const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, 1.0f, k); \
    out[k] = bf16_pair(f[0] * sc, f[1] * sc);                                \
  } while (0)
__device__ __forceinline__ void fp4x8_to_bf16_nv(uint32_t packed, float sc, uint32_t out[4]) {
  MXS_NV_PAIR(0);
  MXS_NV_PAIR(1);
  MXS_NV_PAIR(2);
  MXS_NV_PAIR(3);
}
#undef MXS_NV_PAIR

// The same as four f16 pairs, for the f16 MFMA: the codes widen exactly to
// f16 (v_cvt_scalef32_pk_f16_fp4 with scale 1) and one packed f16 multiply
// applies the block scale (sc: the e4m3 value in both halves); the product is
// exact in f16 too (<= 6 significant bits, 2^-10 .. 2688, all normal).
#define MXS_NV16_PAIR(k)                                                                                   \
  out[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, k) * sc)
__device__ __forceinline__ void fp4x8_to_f16_nv(uint32_t packed, f16x2 sc, uint32_t out[4]) {
  MXS_NV16_PAIR(0);
  MXS_NV16_PAIR(1);
  MXS_NV16_PAIR(2);
  MXS_NV16_PAIR(3);
}
#undef MXS_NV16_PAIR

// Four e4m3 codes (one dword) -> two dwords of bf16 pairs, element order kept
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, e4m3 has 3 mantissa bits;
// 0x7F / 0xFF give NaN; checked against a bit-level decode on all 256 codes).
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t d) {
  return make_uint2(bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false)),
                    bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true)));
}

// ---------------------------------------------------------------- stores seen across the GPU
// COH: a store that other workgroups of the same launch, on any XCD, read
// after a device-scope counter says it is done (an agent-scope relaxed atomic
// store: the sc1 cache policy, so the value does not wait in this XCD's L2);
// otherwise a plain store (read only by later launches).
template <bool COH>
__device__ __forceinline__ void st_u8(uint8_t *p, uint32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, (uint8_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = (uint8_t)v;
}
template <bool COH>
__device__ __forceinline__ void st_u16(uint16_t *p, uint32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, (uint16_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = (uint16_t)v;
}
template <bool COH>
__device__ __forceinline__ void st_u32(uint32_t *p, uint32_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COH>
__device__ __forceinline__ void st_u64(uint64_t *p, uint64_t v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool COH>
__device__ __forceinline__ void st_f32(float *p, float v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// The XCC (one of the 8 accelerator dies, each with its own L2) this wave
// runs on: the low 3 bits of the hardware register XCC_ID.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 7u;
}

// ---------------------------------------------------------------- wave helpers
// The value lane (lane ^ M) holds, for M a power of two below 64:
//   1, 2: DPP quad permutes; 8: row rotate by 8; 4: row rotates by 4 and 12
//   (lane - 4 for lanes with bit 2 set, lane + 4 otherwise); 16, 32: the
//   gfx950 permlane swaps of a value with itself, which hand each half its
//   partner's copy.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const uint32_t lane = threadIdx.x & 63u;
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false);   // row_ror:4
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x12C, 0xF, 0xF, false);   // row_ror:12
    return (lane & 4u) ? dn : up;
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);   // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16u) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "lane xor mask");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32u) ? r[0] : r[1];
  }
}


}  // namespace mxs
