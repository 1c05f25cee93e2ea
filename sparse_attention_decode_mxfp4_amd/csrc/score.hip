// Index scorer: block scores of every page of the index cache against all
// query rows of a sequence.
//
// Definition (the tiny decode configuration's block score, computed by the
// index scorer of ATOM PR #2812, "Mono decode over the MXFP4 KV and index
// caches", commit message of the MXFP4 index-cache commit):
//   S[b][j][i] = max over t in block i, t <= pos_j, of
//                sum_h w[b][j][h] * max(0, q_idx[b][j][h] . k_idx[t])
//
// The contraction q_idx . k runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16):
// M = query rows x index heads (4 A-rows per query row, heads padded to 4),
// N = 16 tokens, K = head_dim. The page's e2m1 keys are widened to bf16 in
// registers with their e8m0 group scale (v_cvt_scalef32_pk_bf16_fp4; bf16
// holds every e2m1 value times a power of two exactly, so the products are
// exact and only the fp32 accumulation rounds).
//
// Lane layout (lane = 16 kg + n): for an N-tile of 16 tokens the lane takes
// the 16 bytes of token n's group kg — one 32-element group and its one scale
// byte — so a wave's load instruction covers 16 whole token rows (1 KiB,
// coalesced), copied straight into LDS (see dma_page). The MFMA's K index is permuted to match: k-step s, lane group
// kg carries elements 32 kg + 8 s .. 32 kg + 8 s + 7, and the q_idx fragment
// follows the same permutation ("q_frag follows the 32-element groups" in the
// commit message). The result tile gives each lane the 4 index heads of one
// query row for one token, so the head sum, ReLU, weights and causal mask stay
// in the lane, and the block max is a 16-lane reduction per page.
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
//   MXFP4: codes of group kg (16 B) at stage + 1024 nt + 16 lane;
//   FP8:   codes 32 kg .. 32 kg + 31 (2 x 16 B) at stage + 1024 (2 nt + c) + 16 lane.
// The chunk's 256 B of per-token scales follow the codes (4096 or 8192 B in).
template <int FMT> struct Chunk;
template <> struct Chunk<0> { static constexpr int kCodes = 4096, kBytes = 4096 + 256, kDma = 5, kPage = kMxPageBytes, kScale = kMxScaleOff; };
template <> struct Chunk<1> { static constexpr int kCodes = 8192, kBytes = 8192 + 256, kDma = 9, kPage = kF8PageBytes, kScale = kF8ScaleOff; };

// Launch shape per index format: waves per workgroup, pages per wave, LDS
// stages per wave. MXFP4: 4 x 4 x 4 stages of 4.25 KiB = 68 KiB of LDS per
// workgroup, two workgroups per CU, ~100 KiB of copies in flight per CU.
template <int FMT> struct ScoreShape;
template <> struct ScoreShape<0> { static constexpr int kWaves = 4, kPages = 4, kStages = 4; };
template <> struct ScoreShape<1> { static constexpr int kWaves = 4, kPages = 2, kStages = 2; };

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

template <int FMT>
__device__ __forceinline__ void dma_chunk(uint8_t *stage, const uint8_t *page, int h, int n, int kg, int lane) {
  if constexpr (FMT == 0) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + 64 * (64 * h + 16 * nt + n) + 16 * kg),
                                       (lds_ptr_t)(stage + 1024 * nt), 16, 0, 0);
  } else {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
        __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + 128 * (64 * h + 16 * nt + n) + 32 * kg + 16 * cc),
                                         (lds_ptr_t)(stage + 1024 * (2 * nt + cc)), 16, 0, 0);
  }
  __builtin_amdgcn_global_load_lds((glb_ptr_t)(page + Chunk<FMT>::kScale + 256 * h + 4 * lane),
                                   (lds_ptr_t)(stage + Chunk<FMT>::kCodes), 4, 0, 0);
}

// B operand (k-step s) of tile nt: the lane's key elements 32 kg + 8 s .. + 7 as bf16.
template <int FMT>
__device__ __forceinline__ void key_operands(const uint8_t *stage, int nt, int n, int kg, int lane, bf16x8 Bk[4],
                                             float &ksc) {
  if constexpr (FMT == 0) {
    const u32x4 kd = *reinterpret_cast<const u32x4 *>(stage + 1024 * nt + 16 * lane);
    const float sf = e8m0_f32(stage[Chunk<0>::kCodes + 4 * (16 * nt + n) + kg]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t w4[4];
      fp4x8_to_bf16(kd[s], sf, w4);
      Bk[s] = __builtin_bit_cast(bf16x8, u32x4{w4[0], w4[1], w4[2], w4[3]});
    }
    ksc = 1.0f;
  } else {
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u32x4 kd = *reinterpret_cast<const u32x4 *>(stage + 1024 * (2 * nt + cc) + 16 * lane);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint2 x = e4m3x4_to_bf16(kd[2 * hh]), y = e4m3x4_to_bf16(kd[2 * hh + 1]);
        Bk[2 * cc + hh] = __builtin_bit_cast(bf16x8, u32x4{x.x, x.y, y.x, y.y});
      }
    }
    ksc = *reinterpret_cast<const float *>(stage + Chunk<1>::kCodes + 4 * (16 * nt + n));
  }
}

// The decode step's K / V row stores and q pack for sequence b, spread over
// the sequence's NW-wave workgroups (nothing in this launch reads them; the
// attention launch that follows does): row r of the 2q K / V rows goes to wave
// r of the sequence's waves, q element 4i to thread i.
template <int NW>
__device__ __forceinline__ void step_side_stores(const CacheView &c, const StepStore &st, int b, int q, int L,
                                                 int lane, int wave) {
  const int nwg = gridDim.x;
  if (st.k_new) {
    for (int r = blockIdx.x * NW + wave; r < 2 * q; r += nwg * NW) {
      const int j = r % q, t = L - q + j;
      if (t < 0 || t / kTokens >= c.stride) continue;
      const int page = c.page_table[(int64_t)b * c.stride + t / kTokens];
      if (page < 0 || page >= c.num_pages) continue;
      const float *src = (r < q ? st.k_new : st.v_new) + ((int64_t)b * q + j) * kDim;
      uint8_t *pool = r < q ? c.k_pages : c.v_pages;
      const float2 x = reinterpret_cast<const float2 *>(src)[lane];
      if (c.kv_format == 0)
        mx_store_row(x, pool + (int64_t)page * kMxPageBytes, t % kTokens, lane);
      else
        f8_store_row(x, pool + (int64_t)page * kF8PageBytes, t % kTokens, lane);
    }
  }
  if (st.q8) {
    const int64_t n = (int64_t)q * st.H * kDim, base = (int64_t)b * n;
    for (int64_t i = 4 * ((int64_t)blockIdx.x * 64 * NW + threadIdx.x); i < n; i += 4 * (int64_t)nwg * 64 * NW)
      pack_q4(st.q_att, st.q_dtype, base + n, st.q8, base + i);
  }
}

template <int MT, int FMT, int NW, int PPW, int S>
__global__ __launch_bounds__(64 * NW) void k_index_score(CacheView c, const uint16_t *__restrict__ q_idx,
                                                         const float *__restrict__ w, int32_t q, int32_t H_I,
                                                         float *__restrict__ scores, StepStore st) {
  using CK = Chunk<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t stages[NW][S][CK::kBytes];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int p0 = (blockIdx.x * NW + wave) * PPW;
  const float NEG_INF = -__builtin_inff();
  float *srow = scores + (int64_t)b * q * c.stride;
  if (p0 >= c.stride) {                             // the grid's rounding: no pages
    step_side_stores<NW>(c, st, b, q, c.context_lens[b], lane, wave);
    return;
  }

  // ---- prologue, one round trip: the context length, this wave's page ids
  // (clamped to the table row, so every load is unconditional; entries past
  // the context or out of range are masked below), the A operand and weights.
  const int L = c.context_lens[b];
  int raw[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) raw[i] = c.page_table[(int64_t)b * c.stride + min(p0 + i, c.stride - 1)];

  // A operand: q_idx rows m = 16 mt + n -> (query row m / 4, head m % 4); rows
  // past q or H_I are zero (their load reads row 0 and is discarded)
  bf16x8 A[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = 16 * mt + n, jA = m >> 2, hA = m & 3;
    const bool ok = jA < q && hA < H_I;
    const uint16_t *src = q_idx + ((int64_t)b * q * H_I + (ok ? jA * H_I + hA : 0)) * kDim + 32 * kg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4 *>(src + 8 * s);
      if (!ok) v = u32x4{0u, 0u, 0u, 0u};
      A[mt][s] = __builtin_bit_cast(bf16x8, v);
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
  // Consume every prologue load here, so that no compiler-placed wait for them
  // lands inside the chunk pipeline (the compiler does not count the
  // direct-to-LDS copies and would wait for all of them).
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int h = 0; h < 4; ++h) asm volatile("" ::"v"(wv[mt][h]));
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, A[mt][s])));
  }
#pragma unroll
  for (int i = 0; i < PPW; ++i) asm volatile("" ::"v"(raw[i]));
  asm volatile("" ::"s"(L) : "memory");

  const int lim = min((L + kTokens - 1) / kTokens, (int)c.stride);    // pages holding tokens
  if (p0 >= lim) {                                  // past the context: no candidates here
    for (int i = 0; i < PPW && p0 + i < c.stride; ++i)
      if (n == 0)
        for (int jw = kg; jw < q; jw += 4) srow[(int64_t)jw * c.stride + p0 + i] = NEG_INF;
    step_side_stores<NW>(c, st, b, q, L, lane, wave);
    return;
  }
  int phys[PPW];
  bool valid[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    valid[i] = p0 + i < lim && raw[i] >= 0 && raw[i] < c.num_pages;
    phys[i] = valid[i] ? raw[i] : 0;
  }
  int posw[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) posw[mt] = L - q + 4 * mt + kg;
  const int pos_min = L - q;                        // the first query row's position

  // The step's new index rows that fall in this wave's pages are stored here,
  // before the pages are copied; the wave waits for its own stores, which
  // reach L2 before the copies read it (nothing cached them earlier).
  if (st.idx_new && L - 1 >= p0 * kTokens && L - q < (p0 + PPW) * kTokens) {
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      if (!valid[i]) continue;
      for (int j = 0; j < q; ++j) {
        const int t = L - q + j;
        if (t < 0 || t / kTokens != p0 + i) continue;
        const float2 x = reinterpret_cast<const float2 *>(st.idx_new + ((int64_t)b * q + j) * kDim)[lane];
        if constexpr (FMT == 0)
          mx_store_row(x, c.idx_pages + (int64_t)phys[i] * kMxPageBytes, t % kTokens, lane);
        else
          f8_store_row(x, c.idx_pages + (int64_t)phys[i] * kF8PageBytes, t % kTokens, lane);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // ---- the chunk pipeline. The waits are explicit (the compiler does not
  // order LDS reads after direct-to-LDS loads): vmcnt counts this wave's
  // vector memory operations in issue order, so "at most n chunks' copies
  // outstanding" right after issuing chunk u + n means every older operation
  // — chunk u's copies included — is done (younger stores only make the wait
  // longer). Stage (u + S - 1) % S is refilled only after chunk u - 1, which
  // it held, has been computed.
  constexpr int kUnits = 2 * PPW;
#pragma unroll
  for (int u = 0; u < S - 1 && u < kUnits; ++u)
    dma_chunk<FMT>(stages[wave][u], c.idx_pages + (int64_t)phys[u >> 1] * CK::kPage, u & 1, n, kg, lane);
  // the side stores go out while the first copies are in flight
  step_side_stores<NW>(c, st, b, q, L, lane, wave);

  float rmax[MT];
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    const int i = u >> 1, h = u & 1;
    const int p = p0 + i;
    const uint8_t *stage = stages[wave][u % S];
    if (u + S - 1 < kUnits) {
      const int un = u + S - 1;
      dma_chunk<FMT>(stages[wave][un % S], c.idx_pages + (int64_t)phys[un >> 1] * CK::kPage, un & 1, n, kg, lane);
    }
    wait_chunks<CK::kDma, S - 1>(min(S - 1, kUnits - 1 - u));
    if (h == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) rmax[mt] = NEG_INF;
    }
    // tokens of this chunk all at or before every row's position: no mask
    const bool full = p * kTokens + 64 * h + 63 <= pos_min;
#pragma unroll 2
    for (int nt = 0; nt < 4; ++nt) {
      bf16x8 Bk[4];
      float ksc;
      key_operands<FMT>(stage, nt, n, kg, lane, Bk, ksc);
      const int t = p * kTokens + 64 * h + 16 * nt + n;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][s], Bk[s], acc, 0, 0, 0);
        float v = 0.f;
#pragma unroll
        for (int hd = 0; hd < 4; ++hd) v += wv[mt][hd] * relu1(FMT == 1 ? acc[hd] * ksc : acc[hd]);
        rmax[mt] = fmaxf(rmax[mt], (full || t <= posw[mt]) ? v : NEG_INF);
      }
    }
    if (h == 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float r = max16_dpp(rmax[mt]);
        const int jw = 4 * mt + kg;
        if (n == 0 && jw < q && p < c.stride) srow[(int64_t)jw * c.stride + p] = valid[i] ? r : NEG_INF;
      }
    }
  }
}

template <int FMT, int MT>
static void launch_shape(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                         int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  using SH = ScoreShape<FMT>;
  const dim3 grid((unsigned)((c.stride + SH::kWaves * SH::kPages - 1) / (SH::kWaves * SH::kPages)), (unsigned)B);
  hipLaunchKernelGGL((k_index_score<MT, FMT, SH::kWaves, SH::kPages, SH::kStages>), grid, dim3(64 * SH::kWaves), 0,
                     s, c, q_idx, w, q, H_I, scores, st);
}

template <int FMT>
static void launch_fmt(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                       int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  switch ((4 * q + 15) / 16) {                      // M tiles: 4 A-rows per query row
    case 1: launch_shape<FMT, 1>(c, q_idx, w, B, q, H_I, scores, st, s); break;
    case 2: launch_shape<FMT, 2>(c, q_idx, w, B, q, H_I, scores, st, s); break;
    case 3: launch_shape<FMT, 3>(c, q_idx, w, B, q, H_I, scores, st, s); break;
    default: launch_shape<FMT, 4>(c, q_idx, w, B, q, H_I, scores, st, s); break;
  }
}

hipError_t launch_index_score(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B,
                              int32_t q, int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  if (c.idx_format == 0)
    launch_fmt<0>(c, q_idx, w, B, q, H_I, scores, st, s);
  else
    launch_fmt<1>(c, q_idx, w, B, q, H_I, scores, st, s);
  return hipGetLastError();
}

}  // namespace mxs
