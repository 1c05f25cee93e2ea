// Index scorer launches: the launch shape by page count (the device code is in
// score.hpp, shared with the single-launch decode step).
#include "score.hpp"

namespace mxs {

template <int FMT, int MT, class SH>
static void launch_shape(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                         int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  const dim3 grid((unsigned)B, (unsigned)((c.stride + SH::kWaves * SH::kPages - 1) / (SH::kWaves * SH::kPages)));
  hipLaunchKernelGGL((k_index_score<MT, FMT, SH::kWaves, SH::kPages, SH::kStages>), grid, dim3(64 * SH::kWaves), 0,
                     s, c, q_idx, w, q, H_I, scores, st);
}

template <int FMT, int MT>
static void launch_mt(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                      int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  const int64_t pages = (int64_t)B * c.stride;
  if constexpr (FMT == 1) {               // 8.25 KiB chunks: two stages per wave
    // one page per wave below 2048 pages, two waves per workgroup so that the
    // pages spread over every CU (4 sequences x 128 pages: 4.2 us against 5.1 us
    // for four waves per workgroup and 7.2 us for two pages per wave)
    if (pages >= 256 * 8)
      launch_shape<FMT, MT, Shape<4, 2, 2>>(c, q_idx, w, B, q, H_I, scores, st, s);
    else
      launch_shape<FMT, MT, Shape<2, 1, 2>>(c, q_idx, w, B, q, H_I, scores, st, s);
  } else if (pages >= 512 * 32) {         // >= 512 workgroups of 32 pages: two per CU with the longer ones
    // (32 ragged sequences, 8K-256K: step 105.5 against 107.4 us for 4 x 4 x 2,
    // scorer 70.1 against 72.6; 4 sequences x 2048 pages, 256 workgroups of 32
    // pages, ran 32.4 against 29.5 us, so below this size 4 x 4 x 2 stays)
    launch_shape<FMT, MT, Shape<4, 8, 2>>(c, q_idx, w, B, q, H_I, scores, st, s);
  } else if (pages >= 256 * 16) {         // >= 256 workgroups of 16 pages, two per CU (MXFP4; NVFP4 alike)
    launch_shape<FMT, MT, Shape<4, 4, 2>>(c, q_idx, w, B, q, H_I, scores, st, s);
  } else {
    launch_shape<FMT, MT, Shape<4, 1, 2>>(c, q_idx, w, B, q, H_I, scores, st, s);
  }
}

template <int FMT>
static void launch_fmt(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                       int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  switch ((4 * q + 15) / 16) {                      // M tiles: 4 A-rows per query row
    case 1: launch_mt<FMT, 1>(c, q_idx, w, B, q, H_I, scores, st, s); break;
    case 2: launch_mt<FMT, 2>(c, q_idx, w, B, q, H_I, scores, st, s); break;
    case 3: launch_mt<FMT, 3>(c, q_idx, w, B, q, H_I, scores, st, s); break;
    default: launch_mt<FMT, 4>(c, q_idx, w, B, q, H_I, scores, st, s); break;
  }
}

hipError_t launch_index_score(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B,
                              int32_t q, int32_t H_I, float *scores, const StepStore &st, hipStream_t s) {
  if (c.idx_format == 0)
    launch_fmt<0>(c, q_idx, w, B, q, H_I, scores, st, s);
  else if (c.idx_format == 1)
    launch_fmt<1>(c, q_idx, w, B, q, H_I, scores, st, s);
  else
    launch_fmt<2>(c, q_idx, w, B, q, H_I, scores, st, s);
  return hipGetLastError();
}

}  // namespace mxs
