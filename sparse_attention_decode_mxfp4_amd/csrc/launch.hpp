// Internal launchers between the C ABI (api.cpp) and the kernels. Arguments
// are validated by the caller; launchers only size grids and enqueue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxs {

struct CacheView {
  uint8_t *k_pages, *v_pages, *idx_pages;
  int32_t num_pages, kv_format, idx_format;
  const int32_t *page_table;
  int32_t stride;
  const int32_t *context_lens;
};

// Floats per query row of the decode step's partial maxima and sums (sp_m,
// sp_l [rows][stride], head h of partition p at h P + p): H P rounded up to
// 32, so that no two rows share a 128-byte line.
inline __host__ __device__ int step_ml_stride(int H, int P) { return (H * P + 31) & ~31; }

// n words at p set to zero (store.hip)
hipError_t launch_zero(uint32_t *p, size_t n, hipStream_t s);

// row store / q store (store.hip)
hipError_t launch_row_store(int format, const float *rows, int64_t n, const int64_t *slots,
                            uint8_t *pages, int32_t num_pages, hipStream_t s);
hipError_t launch_pack_q(const void *q, int q_dtype, int64_t n, uint8_t *q8, hipStream_t s);
// the stores of a step that reuses a block selection: the new K / V rows of
// [B][q][128] fp32 (row j of sequence b at position L_b - q + j; either null:
// none), the query packed to e4m3 when q8 is non-null, counters [B][q] cleared
hipError_t launch_reuse_store(const CacheView &c, const float *k_new, const float *v_new, const void *q, int q_dtype,
                              int32_t H, uint8_t *q8, uint64_t *counters, int32_t B, int32_t q_rows, hipStream_t s);

// The decode step's own stores, done inside the scorer launch (all null: none):
// the new K / V / index rows [B][q][128] fp32 (row j of sequence b goes to
// position L_b - q + j) and the query packed to e4m3 (q8 non-null).
struct StepStore {
  const float *k_new = nullptr, *v_new = nullptr, *idx_new = nullptr;
  const void *q_att = nullptr;
  int q_dtype = 0, H = 0;
  uint8_t *q8 = nullptr;
  uint64_t *counters = nullptr;      // [B][q] cleared (the attention launch's merge counters)
};

// index scores (score.hip)
hipError_t launch_index_score(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B,
                              int32_t q, int32_t H_I, float *scores, const StepStore &st, hipStream_t s);

// top-k (topk.hip)
hipError_t launch_topk(const CacheView &c, const float *scores, int32_t B, int32_t q, int32_t topk,
                       int32_t *block_table, hipStream_t s);

// split attention (attn.hip)
hipError_t launch_split_attn(const CacheView &c, const void *q, int q_dtype,
                             const int32_t *block_table, int32_t B, int32_t q_rows, int32_t H,
                             int32_t topk, int32_t P, float sm_scale, float *sp_m, float *sp_l,
                             float *sp_o, hipStream_t s);

// the decode step's attention (attn.hip): each workgroup selects its row's
// top-k blocks from the scores [B][q_rows][stride] itself, writes the row's
// block table (partition 0) and attends to its partition's slots; the row's
// last partition to finish merges the row into out / lse (counters [B][q_rows]
// zero on entry; the merging workgroup sets its row's counter back to zero)
struct FusedMerge {
  uint64_t *counters = nullptr;       // [B][q_rows]: arrivals (bits 0-7) and per-XCC arrivals (7 bits each from bit 8)
  uint16_t *out = nullptr;
  float *lse = nullptr;
};
hipError_t launch_select_attn(const CacheView &c, const float *scores, const void *q, int32_t B, int32_t q_rows,
                              int32_t H, int32_t topk, int32_t P, float sm_scale, int32_t *block_table, float *sp_m,
                              float *sp_l, float *sp_o, const FusedMerge &fm, hipStream_t s);
// the same launch over a given block table [B][q_rows][topk] (a reused
// selection: entries < 0, past the table or past the row's position are skipped)
hipError_t launch_table_attn(const CacheView &c, const int32_t *block_table, const void *q, int32_t B, int32_t q_rows,
                             int32_t H, int32_t topk, int32_t P, float sm_scale, float *sp_m, float *sp_l, float *sp_o,
                             const FusedMerge &fm, hipStream_t s);

// the whole decode step as one launch (attn.hip): scoring workgroups (which
// also do the step's row and query stores, device-coherent) and then
// attention workgroups that wait for their sequence's scores. Taken when
// decode_step_one_launch holds (MXFP4 K / V and index caches, q <= 8 query
// rows, B x page_table_stride >= 8192 pages); seq_cnt [B][2] zero on entry and
// left zero; st.counters must be null (the merge counters reset themselves).
bool decode_step_one_launch(const CacheView &c, int32_t B, int32_t q);
hipError_t launch_decode_step(const CacheView &c, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                              int32_t H_I, float *scores, const StepStore &st, int32_t H, int32_t topk, int32_t P,
                              float sm_scale, int32_t *block_table, float *sp_m, float *sp_l, float *sp_o,
                              const FusedMerge &fm, uint32_t *seq_cnt, hipStream_t s);

// the step of a layer that reuses a block selection as one launch (attn.hip):
// store workgroups (the new K / V rows, device-coherent) and then attention
// workgroups over the given block table; the query (fp32 / bf16 per q_dtype)
// is rounded to e4m3 in registers for an MXFP4 KV cache, and only the token
// ranges holding the step's new rows wait for their sequence's stores. The
// merge counters fm.counters [B][q_rows] and seq_cnt [B][2] zero on entry and
// left zero.
hipError_t launch_reuse_step(const CacheView &c, const float *k_new, const float *v_new, const void *q, int q_dtype,
                             const int32_t *block_table, int32_t B, int32_t q_rows, int32_t H, int32_t topk,
                             int32_t P, float sm_scale, float *sp_m, float *sp_l, float *sp_o, const FusedMerge &fm,
                             uint32_t *seq_cnt, hipStream_t s);

// streaming read of every index page in page-table order (read.hip): a
// measurement of the scan's bandwidth ceiling; sink receives at most one word
hipError_t launch_read_pages(const CacheView &c, int32_t B, uint32_t page_bytes, uint32_t *sink, hipStream_t s);

// sets the thread-local message that mxs_last_error() returns and gives back
// `code` (api.cpp; for entry points defined in other sources)
int api_error(int code, const char *msg);

// merge (merge.hip)
hipError_t launch_lse_merge(const float *sp_m, const float *sp_l, const float *sp_o, int32_t n_rows,
                            int32_t P, uint16_t *out, float *lse, hipStream_t s);

}  // namespace mxs
