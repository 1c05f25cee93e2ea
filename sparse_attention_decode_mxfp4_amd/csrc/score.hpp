// Index scorer (device code): block scores of every page of the index cache against all
// query rows of a sequence.
//
// Definition (the tiny decode configuration's block score, computed by the
// index scorer of ATOM PR #2812, "Mono decode over the MXFP4 KV and index
// caches", commit message of the MXFP4 index-cache commit):
//   S[b][j][i] = max over t in block i, t <= pos_j, of
//                sum_h w[b][j][h] * max(0, q_idx[b][j][h] . k_idx[t])
//
// The contraction q_idx . k runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16;
// NVFP4 keys on the f16 one, see query_rows_f16):
// M = query rows x index heads (4 A-rows per query row, heads padded to 4),
// N = 16 tokens, K = head_dim. The page's e2m1 keys are widened to bf16 in
// registers with their e8m0 group scale (v_cvt_scalef32_pk_bf16_fp4; bf16
// holds every e2m1 value times a power of two exactly, so the products are
// exact and only the fp32 accumulation rounds). FP8 keys widen exactly to
// bf16 and NVFP4 keys to bf16 times their e4m3 block scale (exact as well);
// both apply the token's fp32 scale to the dot product.
//
// Lane layout (lane = 16 kg + n): for an N-tile of 16 tokens the lane takes
// the 16 bytes of token n's group kg — one 32-element group and its one scale
// byte — so a wave's load instruction covers 16 whole token rows (1 KiB,
// coalesced), copied straight into LDS (see dma_chunk). The MFMA's K index is
// permuted to match: k-step s, lane group kg carries elements 32 kg + 8 s ..
// 32 kg + 8 s + 7, and the q_idx fragment follows the same permutation (the
// commit message lays the query fragment out along the 32-element groups as
// well). The result tile gives each lane the 4 index heads of one query row
// for one token, so the head sum, ReLU, weights and causal mask stay
// in the lane, and the block max is a 16-lane reduction per page.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "rowstore.hpp"

namespace mxs {

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *glb_ptr_t;

// Chunk staging. A chunk is half a page (64 tokens). Each wave owns a ring of
// S LDS stages and keeps S - 1 chunks in flight: chunk u + S - 1 is copied
// global -> LDS with the direct-to-LDS loads (global_load_lds_dwordx4: 64
// lanes x 16 B land in 1 KiB of LDS in lane order; nothing is held in VGPRs)
// while chunk u is computed. Each lane reads back exactly the bytes it copied.
// Lane (n, kg) of the chunk's tile nt (token 64 h + 16 nt + n of the page,
// h = half):
//   MXFP4, NVFP4: codes of group kg (16 B) at stage + 1024 nt + 16 lane;
//   FP8:   codes 32 kg .. 32 kg + 31 (2 x 16 B) at stage + 1024 (2 nt + c) + 16 lane.
// The chunk's 256 B of per-token scales follow the codes (4096 or 8192 B in);
// NVFP4 puts the 64 tokens' 512 B of e4m3 block scales there (8 per token, in
// page order) and the 256 B of fp32 token scales after them.
template <int FMT> struct Chunk;
template <> struct Chunk<0> { static constexpr int kCodes = 4096, kBytes = 4096 + 256, kDma = 5, kPage = kMxPageBytes, kScale = kMxScaleOff; };
template <> struct Chunk<1> { static constexpr int kCodes = 8192, kBytes = 8192 + 256, kDma = 9, kPage = kF8PageBytes, kScale = kF8ScaleOff; };
template <> struct Chunk<2> { static constexpr int kCodes = 4096, kTok = 4096 + 512, kBytes = 4096 + 512 + 256, kDma = 7, kPage = kNvPageBytes; };

// Launch shapes: waves per workgroup, pages per wave, LDS stages per wave.
// Measured on MI355X, each shape timed in one session at loaded clocks
// (stand-alone scorer / full step): at >= 4096 pages, 4 x 4 x 2 (two
// workgroups per CU) against 4 x 8 x 3 (one per CU): 4 sequences x 2048
// pages 17.6 / 34.2-34.5 us against 17.9 / 34.7, the same over NVFP4 pages
// 21.6 / 39.3-40.1 against 22.1 / 42.7, 32 ragged sequences (8K-256K)
// 80.1 / 115.4 against 85.0 / 122.6; 4 x 2 x 2, 4 x 4 x 3, 4 x 8 x 2 and
// 8 x 4 x 2 were no better anywhere. Smaller page tables want short
// workgroups (512 pages: 4 x 1 x 2 at 6.9 us against 7.1 us for 4 x 2 x 2
// and 9.6 us for 4 x 4 x 2).
template <int NW_, int PPW_, int S_> struct Shape {
  static constexpr int kWaves = NW_, kPages = PPW_, kStages = S_;
};

// s_waitcnt vmcnt(n * D) for a wave-uniform n <= K that is a constant once the
// chunk loop is unrolled: at most the n most recently issued chunks (D copies
// each) still in flight.
template <int D, int K>
__device__ __forceinline__ void wait_chunks(int n) {
  if constexpr (K == 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    if (n >= K)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * D) : "memory");
    else
      wait_chunks<D, K - 1>(n);
  }
}

// max(x, 0) as one integer max on the bits: a negative float is a negative
// int (-> +0), any other value keeps its bits. Unlike fmaxf on an MFMA result
// it needs no NaN canonicalisation in front.
__device__ __forceinline__ float relu1(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}
// max over the 16 lanes sharing lane / 16, through DPP lane swizzles (no LDS):
// xor 1 and xor 2 within a quad, then the half-row and row mirrors
template <int CTRL>
__device__ __forceinline__ float dpp_swizzle(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float max16_dpp(float v) {
  v = fmaxf(v, dpp_swizzle<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_swizzle<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_swizzle<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp_swizzle<0x140>(v));   // row_mirror
  return v;
}

// The page copies are non-temporal (the nt cache policy): a step reads each
// index page once, and a model's layers cycle through far more index pages
// than the caches hold, so keeping them out of the caches loses nothing and
// leaves L2 and the Infinity Cache to the scores, tables and K / V pages the
// attention launch reads next. Measured with cache replicas rotated past the
// 256 MB Infinity Cache (same session, step): 4 sequences x 2048 pages 29.8
// against 31.9 us (stand-alone scorer 15.9 against 17.1 us); MXFP4 65K 18.3
// against 19.3; FP8 16K 15.8 against 16.1, FP8 65K 19.6 against 20.5; NVFP4
// 16K level. (When all the replicas fit in that cache, cached copies were
// 0.2-0.4 us faster on the small workloads.)
constexpr int kStreamPolicy = 2;   // nt

template <int FMT>
__device__ __forceinline__ void dma_chunk(uint8_t *stage, const uint8_t *page, int h, int n, int kg, int lane) {
  // page and stage are wave-uniform; the per-lane part of each address is a
  // 32-bit unsigned offset, so the copies take the scalar-base form
  const uint32_t un = (uint32_t)n, ukg = (uint32_t)kg, ul = (uint32_t)lane, uh = (uint32_t)h;
  if constexpr (FMT == 1) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + (128u * (64u * uh + 16u * nt + un) + 32u * ukg + 16u * cc)),
                                         (lds_ptr_t)(stage + 1024 * (2 * nt + cc)), 16, 0, kStreamPolicy);
  } else {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + (64u * (64u * uh + 16u * nt + un) + 16u * ukg)),
                                       (lds_ptr_t)(stage + 1024 * nt), 16, 0, kStreamPolicy);
  }
  if constexpr (FMT == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + ((uint32_t)kNvBScaleOff + 512u * uh + 256u * c + 4u * ul)),
                                       (lds_ptr_t)(stage + Chunk<2>::kCodes + 256 * c), 4, 0, kStreamPolicy);
    __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + ((uint32_t)kNvTScaleOff + 256u * uh + 4u * ul)),
                                     (lds_ptr_t)(stage + Chunk<2>::kTok), 4, 0, kStreamPolicy);
  } else {
    __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + ((uint32_t)Chunk<FMT>::kScale + 256u * uh + 4u * ul)),
                                     (lds_ptr_t)(stage + Chunk<FMT>::kCodes), 4, 0, kStreamPolicy);
  }
}

// The LDS bytes of tile nt that a lane widens: its codes and scales.
template <int FMT> struct KeyRaw;
template <> struct KeyRaw<0> { u32x4 kd; uint32_t sb; };
template <> struct KeyRaw<1> { u32x4 kd[2]; float ksc; };
template <> struct KeyRaw<2> { u32x4 kd; uint32_t bs; float ksc; };

template <int FMT>
__device__ __forceinline__ void key_load(const uint8_t *stage, int nt, int n, int kg, int lane, KeyRaw<FMT> &r) {
  if constexpr (FMT == 0) {
    r.kd = *reinterpret_cast<const u32x4 *>(stage + 1024 * nt + 16 * lane);
    r.sb = stage[Chunk<0>::kCodes + 4 * (16 * nt + n) + kg];
  } else if constexpr (FMT == 2) {
    r.kd = *reinterpret_cast<const u32x4 *>(stage + 1024 * nt + 16 * lane);
    r.bs = *reinterpret_cast<const uint16_t *>(stage + Chunk<2>::kCodes + 8 * (16 * nt + n) + 2 * kg);
    r.ksc = *reinterpret_cast<const float *>(stage + Chunk<2>::kTok + 4 * (16 * nt + n));
  } else {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) r.kd[cc] = *reinterpret_cast<const u32x4 *>(stage + 1024 * (2 * nt + cc) + 16 * lane);
    r.ksc = *reinterpret_cast<const float *>(stage + Chunk<1>::kCodes + 4 * (16 * nt + n));
  }
}

// B operand (k-step s) of a tile: the lane's key elements 32 kg + 8 s .. + 7
// as bf16 (MXFP4, FP8) or f16 (NVFP4) bits.
template <int FMT>
__device__ __forceinline__ void key_widen(const KeyRaw<FMT> &r, u32x4 Bk[4], float &ksc) {
  if constexpr (FMT == 0) {
    const float sf = e8m0_f32(r.sb);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t w4[4];
      fp4x8_to_bf16(r.kd[s], sf, w4);
      Bk[s] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
    ksc = 1.0f;
  } else if constexpr (FMT == 2) {
    // the e4m3 scales of blocks 2 kg and 2 kg + 1 of the lane's token, as f16 (exact)
    const f16x2 bs = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.bs, 1.0f, false);
    const f16x2 s0 = {bs.x, bs.x}, s1 = {bs.y, bs.y};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t w4[4];
      fp4x8_to_f16_nv(r.kd[s], s < 2 ? s0 : s1, w4);
      Bk[s] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
    ksc = r.ksc;
  } else {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint2 x = e4m3x4_to_bf16(r.kd[cc][2 * hh]), y = e4m3x4_to_bf16(r.kd[cc][2 * hh + 1]);
        Bk[2 * cc + hh] = u32x4{x.x, x.y, y.x, y.y};
      }
    }
    ksc = r.ksc;
  }
}

// NVFP4 keys take the f16 MFMA: their widening is then one convert and one
// packed multiply per pair (bf16 has no packed multiply here, and the scaled
// converts apply only a power of two). The query rows become f16 once per
// workgroup: each A row (query row, index head) times 2^e, e chosen so that
// its largest magnitude lies in [2^14, 2^15) (e clamped to [-113, 126] at the
// ends of the bf16 range). bf16 carries 8 significant bits and f16 11, so
// every element of at least 2^-28 times its row's largest lands in f16's
// normal range and converts exactly; a smaller one becomes an f16 subnormal
// (steps of 2^-24 in the scaled units), off by less than 2^-38 of the row's
// largest. The weights of the result rows
// take 2^-e back (a power of two: exact), so the scores are those of the
// bf16 query to that precision. A holds bf16 bits on entry, f16 bits after.
template <int MT>
__device__ __forceinline__ void query_rows_f16(u32x4 (&A)[MT][4], float (&wv)[MT][4], int n, int kg) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    uint32_t a = 0u;                                 // the row's largest |q| (fp32 bits order like values)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) a = max(a, max((A[mt][s][k] << 16) & 0x7FFFFFFFu, A[mt][s][k] & 0x7FFF0000u));
    a = max(a, xor_lane<16>(a));                     // the 4 lane groups hold the row's 128 elements
    a = max(a, xor_lane<32>(a));
    const int e = a == 0u ? 0 : min(max(141 - (int)(a >> 23), -113), 126);
    const float f = u2f((uint32_t)(127 + e) << 23);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t d = A[mt][s][k];
        const f16x2 h = {(_Float16)(u2f(d << 16) * f), (_Float16)(u2f(d & 0xFFFF0000u) * f)};
        A[mt][s][k] = __builtin_bit_cast(uint32_t, h);
      }
    // result rows 16 mt + 4 kg + i are A rows 16 mt + n' with n' = 4 kg + i: lane n' holds their e
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ei = __shfl(e, 4 * kg + i);
      wv[mt][i] *= u2f((uint32_t)(127 - ei) << 23);
    }
  }
  (void)n;
}

// The decode step's new K / V / index rows and e4m3 query, spread over the
// sequence's scoring waves: wave gw (of n_waves) stores rows r = gw + k
// n_waves of the 3q new rows (r < q: K row r; < 2q: V row r - q; else index
// row r - 2q; row j goes to position L - q + j) and packs query elements
// 64 (gw + k n_waves) + lane. The first round's sources are requested in the
// scorer's prologue and stored after the wave's last chunk, so the copies
// never wait for them; later rounds (page tables too short to give every row
// a wave) load and store at the end. Nothing in this launch reads the K / V
// rows or the query; the index rows are scored from the wave that holds
// their positions (see the kernel).
struct SideWork {
  float2 row = make_float2(0.f, 0.f);  // row gw, this lane's two elements
  int page = -1;                       // its page (-1: none)
  float qe = 0.f;                      // query element 64 gw + lane
};

__device__ __forceinline__ int side_rows(const StepStore &st, int q) {
  return (st.k_new ? 2 * q : 0) + (st.idx_new ? q : 0);
}

// row r's source (K, V and index rows are numbered on when present)
__device__ __forceinline__ const float *side_src(const StepStore &st, int b, int q, int r) {
  const float *base = st.k_new ? (r < q ? st.k_new : (r < 2 * q ? st.v_new : st.idx_new)) : st.idx_new;
  return base + ((int64_t)b * q + r % q) * kDim;
}

__device__ __forceinline__ int side_page(const CacheView &c, int b, int q, int L, int r) {
  const int t = L - q + r % q;
  if (t < 0 || t / kTokens >= c.stride) return -1;
  return c.page_table[(int64_t)b * c.stride + t / kTokens];
}

template <bool COH>
__device__ __forceinline__ void side_row(const CacheView &c, const StepStore &st, int b, int q, int L, int r,
                                         float2 x, int page, int lane) {
  const int t = L - q + r % q;
  if (page < 0 || page >= c.num_pages) return;
  const bool kv = st.k_new && r < 2 * q;
  uint8_t *pool = kv ? (r < q ? c.k_pages : c.v_pages) : c.idx_pages;
  store_row<COH>(kv ? c.kv_format : c.idx_format, x, pool, page, t % kTokens, lane);
}

// first-round sources (no dependence on the context length)
__device__ __forceinline__ void side_prefetch(const StepStore &st, int b, int q, int gw, int lane, SideWork &sw) {
  if (gw < side_rows(st, q)) sw.row = reinterpret_cast<const float2 *>(side_src(st, b, q, gw))[lane];
  if (st.q8) {
    const int64_t n = (int64_t)q * st.H * kDim, i = 64 * (int64_t)gw + lane;
    if (i < n) sw.qe = load_q_elem(st.q_att, st.q_dtype, (int64_t)b * n + i);
  }
}

template <bool COH>
__device__ __forceinline__ void side_finish(const CacheView &c, const StepStore &st, int b, int q, int L, int gw,
                                            int n_waves, int lane, const SideWork &sw) {
  const int nr = side_rows(st, q);
  if (gw < nr) side_row<COH>(c, st, b, q, L, gw, sw.row, sw.page, lane);
  for (int r = gw + n_waves; r < nr; r += n_waves)
    side_row<COH>(c, st, b, q, L, r, reinterpret_cast<const float2 *>(side_src(st, b, q, r))[lane],
                  side_page(c, b, q, L, r), lane);
  if (st.q8) {
    const int64_t n = (int64_t)q * st.H * kDim, base = (int64_t)b * n;
    int64_t i = 64 * (int64_t)gw + lane;
    if (i < n) st_u8<COH>(st.q8 + base + i, e4m3_code(sw.qe));
    for (i += 64 * (int64_t)n_waves; i < n; i += 64 * (int64_t)n_waves)
      st_u8<COH>(st.q8 + base + i, e4m3_code(load_q_elem(st.q_att, st.q_dtype, base + i)));
  }
}

// A new row quantized by one wave (this lane: elements 2 lane, 2 lane + 1):
// code = the lane's code byte (MXFP4, NVFP4) or byte pair (FP8); word = the
// token's scale dwords as the page holds them (MXFP4: the four group bytes;
// FP8: the fp32 scale bits; NVFP4: the eight block scale codes, then the fp32
// token scale bits).
template <int FMT> constexpr int kRowWords = FMT == 2 ? 3 : 1;
template <int FMT>
__device__ __forceinline__ void quant_row(float2 x, uint32_t &code, uint32_t (&word)[kRowWords<FMT>]) {
  if constexpr (FMT == 0) {
    uint32_t gsb;
    mx_quant_row(x, code, gsb);
    word[0] = mx_scale_word(gsb);
  } else if constexpr (FMT == 1) {
    float scale;
    f8_quant_row(x, code, scale);
    word[0] = f2u(scale);
  } else {
    uint32_t cb;
    float S;
    nv_quant_row(x, code, cb, S);
    const uint2 w = nv_scale_words(cb);
    word[0] = w.x;
    word[1] = w.y;
    word[2] = f2u(S);
  }
}

// The quantized row into token tc of a chunk held in LDS in the copy layout
// (see the chunk staging above). Called only once the chunk's copy has
// landed (the explicit wait before it): the LDS writes are issued as plain
// instructions, which the compiler would otherwise hold back behind every
// copy still in flight; a wave's LDS operations execute in order, so the
// chunk's reads that follow see them.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)const_cast<uint8_t *>(p);
}
template <int FMT>
__device__ __forceinline__ void patch_row(uint8_t *stage, int tc, uint32_t code, const uint32_t *word, int lane) {
  const int nt = tc >> 4, nn = tc & 15;
  if constexpr (FMT == 0) {
    asm volatile("ds_write_b8 %0, %1" ::"v"(lds_addr(stage + 1024 * nt + 256 * (lane >> 4) + 16 * nn + (lane & 15))),
                 "v"(code) : "memory");
    if (lane == 0)
      asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(stage + Chunk<0>::kCodes + 4 * tc)), "v"(word[0]) : "memory");
  } else if constexpr (FMT == 2) {
    asm volatile("ds_write_b8 %0, %1" ::"v"(lds_addr(stage + 1024 * nt + 256 * (lane >> 4) + 16 * nn + (lane & 15))),
                 "v"(code) : "memory");
    if (lane == 0) {
      asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(stage + Chunk<2>::kCodes + 8 * tc)), "v"(word[0]) : "memory");
      asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(stage + Chunk<2>::kCodes + 8 * tc + 4)), "v"(word[1])
                   : "memory");
      asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(stage + Chunk<2>::kTok + 4 * tc)), "v"(word[2]) : "memory");
    }
  } else {
    asm volatile("ds_write_b16 %0, %1" ::"v"(lds_addr(stage + 1024 * (2 * nt + ((lane & 15) >> 3)) +
                                                        16 * (16 * (lane >> 4) + nn) + 2 * (lane & 7))),
                 "v"(code) : "memory");
    if (lane == 0)
      asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(stage + Chunk<1>::kCodes + 4 * tc)), "v"(word[0]) : "memory");
  }
}

// LDS bytes of one scoring workgroup: the waves' stage rings, then the step's
// new index rows quantized (4 MT rows: 64 lane words, then the scale words).
template <int MT, int FMT, int NW, int S>
constexpr int kScoreLds = NW * S * Chunk<FMT>::kBytes + 4 * MT * (64 + kRowWords<FMT>) * 4;

// One scoring workgroup: sequence b, wave group gy of ny. lds: kScoreLds bytes,
// 16-byte aligned, the workgroup's only LDS object while it scores (a second
// one makes the compiler wait for every copy in flight before any LDS read).
// COH: the scores, the step's stored rows and the e4m3 query are written with
// device-coherent stores (read by other workgroups of the same launch).
template <int MT, int FMT, int NW, int PPW, int S, bool COH>
__device__ __forceinline__ void index_score_wg(const CacheView &c, const uint16_t *__restrict__ q_idx,
                                               const float *__restrict__ w, int32_t q, int32_t H_I,
                                               float *__restrict__ scores, const StepStore &st, int b, int gy, int ny,
                                               uint8_t *lds) {
  using CK = Chunk<FMT>;
  constexpr int kUnits = 2 * PPW;
  static_assert(S >= 2 && S - 1 <= kUnits, "stage ring");
  auto stage_at = [&](int w, int u) { return lds + (w * S + u) * CK::kBytes; };
  uint32_t *s_qc = reinterpret_cast<uint32_t *>(lds + NW * S * CK::kBytes);   // [4 MT][64]
  uint32_t *s_qw = s_qc + 4 * MT * 64;                                        // [4 MT][kRowWords]
  // grid (sequence, wave group). Waves are numbered in dispatch order, d, and
  // take the sequence's pages from the back (d = 0: the last pages, where the
  // step's new rows are, so the wave with the most extra work starts first);
  // the side stores go to the next waves dispatched.
  // The wave index as a wave-uniform (scalar) value: page bases, LDS stage
  // addresses and the side-work indices then live in SGPRs (4 sequences x
  // 2048 pages: step 31.8 against 32.2 us; 32 ragged sequences 112.0
  // against 114.1 us, one session). The two-wave workgroups of small FP8 page
  // tables measured slower that way (step 16.5 against 16.1 us) and keep the
  // vector form.
  const int lane = threadIdx.x & 63;
  const int wave = NW == 2 ? (int)(threadIdx.x >> 6) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int n_waves = ny * NW, d = gy * NW + wave;
  const int gw = (d + n_waves - 1) % n_waves;        // side-store index: d = 1, 2, ... first
  const int p0 = (n_waves - 1 - d) * PPW;
  const float NEG_INF = -__builtin_inff();
  float *srow = scores + (int64_t)b * q * c.stride;

  // ---- prologue, one round trip: the context length, this wave's page ids
  // (clamped to the table row, so every load is unconditional; entries past
  // the context or out of range are masked below), the A operand, the weights
  // and the wave's share of the step's side stores.
  static_assert((PPW & (PPW - 1)) == 0 && PPW <= 64, "pages per wave: a power of two");
  const int L = c.context_lens[b];
  const int pk = lane & (PPW - 1);                   // lane k holds page p0 + k's id
  const int praw = c.page_table[(int64_t)b * c.stride + min(p0 + pk, c.stride - 1)];

  // A operand: q_idx rows m = 16 mt + n -> (query row m / 4, head m % 4); rows
  // past q or H_I are zero (their load reads row 0 and is discarded)
  u32x4 A[MT][4];                                    // bf16 bits (f16 for NVFP4 keys, below)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + n, jA = m >> 2, hA = m & 3;
    const bool ok = jA < q && hA < H_I;
    const uint16_t *src = q_idx + ((int64_t)b * q * H_I + (ok ? jA * H_I + hA : 0)) * kDim + 32 * kg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(src + 8 * s);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      A[mt][s] = v;
    }
  }
  // result rows 16 mt + 4 kg + i -> query row 4 mt + kg, index head i
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int jw = 4 * mt + kg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = jw < q && i < H_I;
      const float x = w[(int64_t)b * q * H_I + (ok ? jw * H_I + i : 0)];
      wv[mt][i] = ok ? x : 0.0f;
    }
  }
  SideWork sw;
  side_prefetch(st, b, q, gw, lane, sw);
  // The step's new index rows are quantized by the waves of the workgroup
  // that holds their positions (rows j = wave + NW k each, into LDS; every
  // wave of it, on either path below, so the barrier sees all of them). That
  // workgroup is known once L (a scalar load, back well before the vector
  // loads above) arrives; only its waves request the rows, so the other
  // workgroups never wait for them.
  const int wg_p0 = (n_waves - NW * (gy + 1)) * PPW;                  // the workgroup's first page
  const bool own_wg = st.idx_new != nullptr && L >= 1 && L - 1 >= wg_p0 * kTokens &&
                      max(L - q, 0) < (wg_p0 + NW * PPW) * kTokens;     // uniform over the workgroup
  constexpr int kOwnRows = (4 * MT + NW - 1) / NW;
  float2 xr[kOwnRows];
  if (own_wg) {
#pragma unroll
    for (int k = 0; k < kOwnRows; ++k)
      xr[k] = reinterpret_cast<const float2 *>(st.idx_new + ((int64_t)b * q + min(wave + NW * k, q - 1)) * kDim)[lane];
#pragma unroll
    for (int k = 0; k < kOwnRows; ++k) asm volatile("" ::"v"(xr[k].x), "v"(xr[k].y));
  }
  // Consume every prologue load here, so that no compiler-placed wait for them
  // lands inside the chunk pipeline (the compiler does not count the
  // direct-to-LDS copies and would wait for all of them).
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int h = 0; h < 4; ++h) asm volatile("" ::"v"(wv[mt][h]));
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(A[mt][s]));
  }
  asm volatile("" ::"v"(praw));
  asm volatile("" ::"v"(sw.row.x), "v"(sw.row.y), "v"(sw.qe));
  asm volatile("" ::"s"(L) : "memory");
  if constexpr (FMT == 2) query_rows_f16<MT>(A, wv, n, kg);

  const int lim = min((L + kTokens - 1) / kTokens, (int)c.stride);    // pages holding tokens
  auto quant_share = [&]() {
    if (!own_wg) return;
#pragma unroll
    for (int k = 0; k < kOwnRows; ++k) {
      const int j = wave + NW * k;
      if (j >= 4 * MT) continue;
      uint32_t code, word[kRowWords<FMT>];
      quant_row<FMT>(xr[k], code, word);
      s_qc[64 * j + lane] = code;
      if (lane == 0)
#pragma unroll
        for (int i = 0; i < kRowWords<FMT>; ++i) s_qw[kRowWords<FMT> * j + i] = word[i];
    }
    // LDS writes done, then the workgroup barrier (no wait for the copies)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  if (gw < side_rows(st, q)) sw.page = side_page(c, b, q, L, gw);
  if (p0 >= lim) {                                  // past the context (or the table): no candidates here
    quant_share();
    if (n == 0)
      for (int i = 0; i < PPW && p0 + i < c.stride; ++i)
        for (int jw = kg; jw < q; jw += 4) st_f32<COH>(srow + (int64_t)jw * c.stride + p0 + i, NEG_INF);
  } else {
    // page p0 + i: valid (inside the context, id in range) = bit i of vmask,
    // its id = lane i's praw (uniform reads, so no per-page registers)
    const uint64_t vmask = __ballot(p0 + pk < lim && praw >= 0 && praw < c.num_pages);
    auto valid_of = [&](int i) { return ((vmask >> i) & 1ull) != 0ull; };
    auto phys_of = [&](int i) { return valid_of(i) ? __builtin_amdgcn_readlane(praw, i) : 0; };
    int posw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) posw[mt] = L - q + 4 * mt + kg;
    const int pos_min = L - q;                        // the first query row's position

    // rmax[mt] = max(rmax[mt], the row's score of every token t of chunk (p, h)
    // with t_lo <= t <= hi[mt]) (all tokens when full; always_full, a
    // compile-time flag, drops the mask altogether). tile_max takes one tile
    // of 16 tokens (token t in this lane).
    auto tile_max = [&](auto always_full, const KeyRaw<FMT> &kr, int t, bool full, int t_lo, const int (&hi)[MT],
                        float (&rmax)[MT]) {
      u32x4 Bk[4];
      float ksc;
      key_widen<FMT>(kr, Bk, ksc);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (FMT == 2)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, A[mt][s]),
                                                         __builtin_bit_cast(f16x8, Bk[s]), acc, 0, 0, 0);
          else
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[mt][s]),
                                                          __builtin_bit_cast(bf16x8, Bk[s]), acc, 0, 0, 0);
        }
        float v = 0.f;
#pragma unroll
        for (int hd = 0; hd < 4; ++hd) v += wv[mt][hd] * relu1(FMT != 0 ? acc[hd] * ksc : acc[hd]);
        if constexpr (decltype(always_full)::value)
          rmax[mt] = fmaxf(rmax[mt], v);
        else
          rmax[mt] = fmaxf(rmax[mt], (full || (t >= t_lo && t <= hi[mt])) ? v : NEG_INF);
      }
    };
    auto chunk_max = [&](auto always_full, const uint8_t *stage, int p, int h, bool full, int t_lo,
                         const int (&hi)[MT], float (&rmax)[MT]) {
      // MXFP4: the chunk's LDS reads all go out first, then its four tiles (one
      // LDS wait per chunk instead of one per two tiles; 4 sequences x 2048
      // pages: 17.5 us against 17.9 us per launch, 32 ragged sequences 79.5
      // against 80.5 us, one session). NVFP4 and FP8 tiles widen with more
      // registers and keep the two-tile loop (NVFP4 was 0.6 us slower the
      // other way).
      if constexpr (FMT == 0) {
        KeyRaw<FMT> kr[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) key_load<FMT>(stage, nt, n, kg, lane, kr[nt]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          tile_max(always_full, kr[nt], p * kTokens + 64 * h + 16 * nt + n, full, t_lo, hi, rmax);
      } else {
#pragma unroll 2
        for (int nt = 0; nt < 4; ++nt) {
          KeyRaw<FMT> kr;
          key_load<FMT>(stage, nt, n, kg, lane, kr);
          tile_max(always_full, kr, p * kTokens + 64 * h + 16 * nt + n, full, t_lo, hi, rmax);
        }
      }
    };

    // The wave takes its pages from its last valid one down (page i_last, then
    // i_last - 1, ..., then the pages past the context, which score -inf).
    // The step's new index rows (positions L - q .. L - 1; their stores into
    // the pages are side work) sit in the last valid page(s), so the wave that
    // holds them meets them in its first chunks. Its workgroup's waves
    // quantize them while their first copies are in flight, and the wave
    // writes them over the chunk's LDS copy (in the copy layout) once the copy
    // has landed, before scoring it.
    const int i_last = min(lim - 1 - p0, PPW - 1);
    auto page_of = [&](int o) { return (i_last - o + PPW) % PPW; };   // order o -> page index
    const bool own = st.idx_new != nullptr && L >= 1 && L - 1 >= p0 * kTokens && max(L - q, 0) < (p0 + PPW) * kTokens;

    // ---- the chunk pipeline. The waits are explicit (the compiler does not
    // order LDS reads after direct-to-LDS loads): vmcnt counts this wave's
    // vector memory operations in issue order, so "at most n chunks' copies
    // outstanding" right after issuing chunk u + n means every older operation
    // — chunk u's copies included — is done. Stage (u + S - 1) % S is refilled
    // only after chunk u - 1, which it held, has been computed.
#pragma unroll
    for (int u = 0; u < S - 1; ++u)
      dma_chunk<FMT>(stage_at(wave, u), c.idx_pages + (int64_t)phys_of(page_of(u >> 1)) * CK::kPage, u & 1, n, kg,
                     lane);
    quant_share();
    float rmax[MT];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
      const int i = page_of(u >> 1), h = u & 1;
      const int p = p0 + i;
      uint8_t *stage = stage_at(wave, u % S);
      if (u + S - 1 < kUnits) {
        const int un = u + S - 1;
        dma_chunk<FMT>(stage_at(wave, un % S), c.idx_pages + (int64_t)phys_of(page_of(un >> 1)) * CK::kPage, un & 1,
                       n, kg, lane);
      }
      wait_chunks<CK::kDma, S - 1>(min(S - 1, kUnits - 1 - u));
      if (u < 4 && own) {                            // the new rows are in the first two pages taken
        const int c0 = p * kTokens + 64 * h;         // the chunk's first position
#pragma unroll
        for (int j = 0; j < 4 * MT; ++j) {
          const int t = L - q + j;
          if (j < q && t >= c0 && t <= c0 + 63)
            patch_row<FMT>(stage, t - c0, s_qc[64 * j + lane], s_qw + kRowWords<FMT> * j, lane);
        }
      }
      if (h == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) rmax[mt] = NEG_INF;
      }
      // only a wave's first four chunks can hold tokens past the first query
      // row's position: the last q <= 16 tokens of the context lie in the
      // last valid page, taken first (chunks 0, 1), or also in the second
      // half of the page before it (chunk 3). Later chunks are whole, or lie
      // past the context and are stored as -inf below, so they skip the mask.
      if (u < 4)
        chunk_max(std::false_type{}, stage, p, h, p * kTokens + 64 * h + 63 <= pos_min, INT32_MIN, posw, rmax);
      else
        chunk_max(std::true_type{}, stage, p, h, true, INT32_MIN, posw, rmax);
      if (h == 1) {
        const bool ok = valid_of(i);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float r = max16_dpp(rmax[mt]);
          const int jw = 4 * mt + kg;
          if (n == 0 && jw < q && p < c.stride) st_f32<COH>(srow + (int64_t)jw * c.stride + p, ok ? r : NEG_INF);
        }
      }
    }
  }
  side_finish<COH>(c, st, b, q, L, gw, n_waves, lane, sw);
  // the attention launch's merge counters for sequence b (at the end: in the
  // prologue this would split the kernel-argument loads into two round trips)
  if (st.counters && gy == ny - 1)
    for (int i = threadIdx.x; i < q; i += 64 * NW) st_u64<COH>(st.counters + b * q + i, 0ull);
}

template <int MT, int FMT, int NW, int PPW, int S>
__global__ __launch_bounds__(64 * NW) void k_index_score(CacheView c, const uint16_t *__restrict__ q_idx,
                                                         const float *__restrict__ w, int32_t q, int32_t H_I,
                                                         float *__restrict__ scores, StepStore st) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kScoreLds<MT, FMT, NW, S>];
  index_score_wg<MT, FMT, NW, PPW, S, false>(c, q_idx, w, q, H_I, scores, st, blockIdx.x, blockIdx.y, gridDim.y,
                                             lds);
}

}  // namespace mxs
