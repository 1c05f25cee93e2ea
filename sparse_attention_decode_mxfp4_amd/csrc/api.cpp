// The C ABI of mxsparse (declared in include/mxsparse.h): host-side argument
// validation, workspace carving and the launch chain of decode_step.
// Every check runs before anything is enqueued, so an error return means no
// work was launched.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "launch.hpp"
#include "mxsparse.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MXS_OK;
}

}  // namespace

namespace mxs {
int api_error(int code, const char *msg) { return fail(code, "%s", msg); }
}  // namespace mxs

namespace {

int launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MXS_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQ(cond, code, ...)            \
  do {                                  \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

size_t page_bytes(int fmt) {
  return fmt == MXS_FMT_MXFP4 ? MXS_MXFP4_PAGE_BYTES : (fmt == MXS_FMT_FP8 ? MXS_FP8_PAGE_BYTES : MXS_NVFP4_PAGE_BYTES);
}

int check_format(int fmt, const char *name) {
  REQ(fmt == MXS_FMT_MXFP4 || fmt == MXS_FMT_FP8 || fmt == MXS_FMT_NVFP4, MXS_EUNSUPPORTED,
      "%s: format %d is not supported (MXFP4 = 0, FP8 = 1 and NVFP4 = 2 are)", name, fmt);
  return MXS_OK;
}

// Validates the parts of the cache a stage reads.
int check_cache(const mxs_cache *c, bool need_idx, bool need_kv) {
  REQ(c, MXS_EINVAL, "cache: null");
  REQ(c->num_pages >= 1, MXS_EINVAL, "cache.num_pages: %d, must be >= 1", c->num_pages);
  REQ(c->page_table, MXS_EINVAL, "cache.page_table: null");
  REQ(c->context_lens, MXS_EINVAL, "cache.context_lens: null");
  REQ(c->page_table_stride >= 1, MXS_EINVAL, "cache.page_table_stride: %d, must be >= 1", c->page_table_stride);
  REQ(c->page_table_stride <= MXS_MAX_PAGES_PER_SEQ, MXS_EUNSUPPORTED,
      "cache.page_table_stride: %d pages per sequence, more than %d", c->page_table_stride, MXS_MAX_PAGES_PER_SEQ);
  if (need_idx) {
    if (int r = check_format(c->idx_format, "cache.idx_format")) return r;
    REQ(c->idx_pages, MXS_EINVAL, "cache.idx_pages: null");
    REQ(aligned(c->idx_pages, 16), MXS_EINVAL, "cache.idx_pages: not 16-byte aligned");
  }
  if (need_kv) {
    if (int r = check_format(c->kv_format, "cache.kv_format")) return r;
    REQ(c->k_pages && c->v_pages, MXS_EINVAL, "cache.k_pages / v_pages: null");
    REQ(aligned(c->k_pages, 16) && aligned(c->v_pages, 16), MXS_EINVAL, "cache.k_pages / v_pages: not 16-byte aligned");
  }
  return MXS_OK;
}

int check_rows(int32_t B, int32_t q) {
  REQ(B >= 0, MXS_EINVAL, "B: %d, must be >= 0", B);
  REQ(q >= 1, MXS_EINVAL, "q: %d, must be >= 1", q);
  REQ(q <= MXS_MAX_Q, MXS_EUNSUPPORTED, "q: %d query rows per sequence, more than %d", q, MXS_MAX_Q);
  return MXS_OK;
}

int check_topk(int32_t topk) {
  REQ(topk >= 1, MXS_EINVAL, "topk: %d, must be >= 1", topk);
  REQ(topk <= MXS_MAX_TOPK, MXS_EUNSUPPORTED, "topk: %d, more than %d", topk, MXS_MAX_TOPK);
  return MXS_OK;
}

mxs::CacheView view(const mxs_cache *c) {
  return mxs::CacheView{c->k_pages, c->v_pages, c->idx_pages, c->num_pages, c->kv_format, c->idx_format,
                        c->page_table, c->page_table_stride, c->context_lens};
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

// Partitions per query row when the caller leaves the choice to the library,
// for every K / V format: one block per wave of a 4-wave partition workgroup
// (ceil(topk / 4)), but no more than it takes to give each of MI355X's 256
// CUs one workgroup. If that leaves CUs without a workgroup, two blocks per
// workgroup instead (ceil(topk / 2), within the same cap): its 4 waves then
// take half blocks (the attention kernels' step_tiles), so every wave still
// works and twice as many workgroups share the rows. Every workgroup runs the
// same dependent chain (selection, block loads, exchange of partials), so
// when the rows alone fill the GPU, fewer and longer partitions beat several
// rounds of short ones. Measured on MI355X (step): top-k 16 over 4 x 8 MXFP4
// rows 18.1 us at P = 8 (half blocks) against 18.4 at P = 4, over NVFP4 rows
// 19.1 against 20.3, over 4 x 4 FP8 rows 15.2 against 16.2 with whole blocks
// at the same P = 8; top-k 32 over 4 x 8 rows keeps P = 8 with whole blocks
// (32.5 us; 35.0 at P = 16 with half blocks).
constexpr int64_t kTargetWorkgroups = 256;
int default_partitions(int32_t B, int32_t q_rows, int32_t topk) {
  const int64_t rows = (int64_t)B * q_rows;
  const int64_t cap = rows > 0 ? std::max<int64_t>(1, kTargetWorkgroups / rows) : MXS_MAX_PARTITIONS;
  int64_t p = std::min<int64_t>((topk + 3) / 4, cap);
  if (p * rows < kTargetWorkgroups) p = std::min<int64_t>((topk + 1) / 2, cap);
  return (int)std::max<int64_t>(1, std::min<int64_t>(p, MXS_MAX_PARTITIONS));
}

// workspace segments of decode_step, in order
struct StepWs {
  size_t scores, table, q8, sp_m, sp_l, sp_o, counters, seq_cnt, total;
};

StepWs step_ws(int32_t B, int32_t q, int32_t H, int32_t topk, int32_t stride, int32_t P) {
  StepWs w;
  const size_t rows = (size_t)B * q;
  size_t off = 0;
  w.scores = off; off += round_up(rows * stride * sizeof(float));
  w.table = off;  off += round_up(rows * topk * sizeof(int32_t));
  w.q8 = off;     off += round_up(rows * H * MXS_HEAD_DIM);
  w.sp_m = off;   off += round_up(rows * mxs::step_ml_stride(H, P) * sizeof(float));
  w.sp_l = off;   off += round_up(rows * mxs::step_ml_stride(H, P) * sizeof(float));
  w.sp_o = off;   off += round_up(rows * H * P * MXS_HEAD_DIM * sizeof(float));
  w.counters = off; off += round_up(rows * sizeof(uint64_t));
  w.seq_cnt = off;  off += round_up((size_t)B * 2 * sizeof(uint32_t));
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

const char *mxs_status_str(int status) {
  switch (status) {
    case MXS_OK: return "ok";
    case MXS_EINVAL: return "invalid argument";
    case MXS_EUNSUPPORTED: return "unsupported configuration";
    case MXS_EWORKSPACE: return "workspace too small";
    case MXS_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char *mxs_last_error(void) { return g_err; }

int mxs_abi_version(void) { return MXS_ABI_VERSION; }

static int row_store(int fmt, const float *rows, int64_t n, const int64_t *slots, uint8_t *pages, int32_t num_pages,
                     void *stream, const char *name) {
  REQ(n >= 0, MXS_EINVAL, "%s: n = %lld, must be >= 0", name, (long long)n);
  REQ(num_pages >= 1, MXS_EINVAL, "%s: num_pages = %d, must be >= 1", name, num_pages);
  REQ(pages && aligned(pages, 16), MXS_EINVAL, "%s: pages null or not 16-byte aligned", name);
  if (n > 0) {
    REQ(rows && aligned(rows, 8), MXS_EINVAL, "%s: rows null or not 8-byte aligned", name);
    REQ(slots && aligned(slots, 8), MXS_EINVAL, "%s: slots null or not 8-byte aligned", name);
  }
  return launched(mxs::launch_row_store(fmt, rows, n, slots, pages, num_pages, (hipStream_t)stream), name);
}

int mxfp4_row_store(const float *rows, int64_t n, const int64_t *slots, uint8_t *pages, int32_t num_pages,
                    void *stream) {
  return row_store(MXS_FMT_MXFP4, rows, n, slots, pages, num_pages, stream, "mxfp4_row_store");
}

int fp8_row_store(const float *rows, int64_t n, const int64_t *slots, uint8_t *pages, int32_t num_pages,
                  void *stream) {
  return row_store(MXS_FMT_FP8, rows, n, slots, pages, num_pages, stream, "fp8_row_store");
}

int nvfp4_row_store(const float *rows, int64_t n, const int64_t *slots, uint8_t *pages, int32_t num_pages,
                    void *stream) {
  return row_store(MXS_FMT_NVFP4, rows, n, slots, pages, num_pages, stream, "nvfp4_row_store");
}

int pack_q_e4m3(const void *q, int32_t q_dtype, int64_t n, uint8_t *q8, void *stream) {
  REQ(q_dtype == MXS_F32 || q_dtype == MXS_BF16, MXS_EUNSUPPORTED, "pack_q_e4m3: q_dtype %d (fp32 or bf16 only)",
      q_dtype);
  REQ(n >= 0, MXS_EINVAL, "pack_q_e4m3: n = %lld, must be >= 0", (long long)n);
  if (n > 0) {
    REQ(q && aligned(q, q_dtype == MXS_F32 ? 4 : 2), MXS_EINVAL, "pack_q_e4m3: q null or misaligned");
    REQ(q8, MXS_EINVAL, "pack_q_e4m3: q8 null");
  }
  return launched(mxs::launch_pack_q(q, q_dtype, n, q8, (hipStream_t)stream), "pack_q_e4m3");
}

static int check_score_args(const mxs_cache *cache, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                            int32_t H_I) {
  if (int r = check_cache(cache, true, false)) return r;
  if (int r = check_rows(B, q)) return r;
  REQ(H_I >= 1, MXS_EINVAL, "H_I: %d, must be >= 1", H_I);
  REQ(H_I <= MXS_MAX_H_I, MXS_EUNSUPPORTED, "H_I: %d index heads, more than %d", H_I, MXS_MAX_H_I);
  REQ(q_idx && aligned(q_idx, 16), MXS_EINVAL, "q_idx: null or not 16-byte aligned");
  REQ(w && aligned(w, 4), MXS_EINVAL, "w: null or misaligned");
  return MXS_OK;
}

int index_score(const mxs_cache *cache, const uint16_t *q_idx, const float *w, int32_t B, int32_t q, int32_t H_I,
                float *scores, void *stream) {
  if (int r = check_score_args(cache, q_idx, w, B, q, H_I)) return r;
  REQ(scores && aligned(scores, 4), MXS_EINVAL, "scores: null or misaligned");
  if (B == 0) return ok();
  return launched(mxs::launch_index_score(view(cache), q_idx, w, B, q, H_I, scores, mxs::StepStore{},
                                          (hipStream_t)stream),
                  "index_score");
}

int topk_blocks(const mxs_cache *cache, const float *scores, int32_t B, int32_t q, int32_t topk,
                int32_t *block_table, void *stream) {
  REQ(cache, MXS_EINVAL, "cache: null");
  REQ(cache->context_lens, MXS_EINVAL, "cache.context_lens: null");
  REQ(cache->page_table_stride >= 1 && cache->page_table_stride <= MXS_MAX_PAGES_PER_SEQ, MXS_EUNSUPPORTED,
      "cache.page_table_stride: %d, must be in 1..%d", cache->page_table_stride, MXS_MAX_PAGES_PER_SEQ);
  if (int r = check_rows(B, q)) return r;
  if (int r = check_topk(topk)) return r;
  REQ(scores && aligned(scores, 4), MXS_EINVAL, "scores: null or misaligned");
  REQ(block_table && aligned(block_table, 4), MXS_EINVAL, "block_table: null or misaligned");
  if (B == 0) return ok();
  return launched(mxs::launch_topk(view(cache), scores, B, q, topk, block_table, (hipStream_t)stream), "topk_blocks");
}

size_t mxs_score_workspace_bytes(int32_t B, int32_t q, int32_t page_table_stride) {
  if (B < 0 || q < 0 || page_table_stride < 0) return 0;
  return round_up((size_t)B * q * page_table_stride * sizeof(float));
}

int index_score_topk(const mxs_cache *cache, const uint16_t *q_idx, const float *w, int32_t B, int32_t q,
                     int32_t H_I, int32_t topk, int32_t *block_table, float *scores, void *ws, size_t ws_bytes,
                     void *stream) {
  if (int r = check_score_args(cache, q_idx, w, B, q, H_I)) return r;
  if (int r = check_topk(topk)) return r;
  REQ(block_table && aligned(block_table, 4), MXS_EINVAL, "block_table: null or misaligned");
  float *sc = scores;
  if (!sc) {
    const size_t need = mxs_score_workspace_bytes(B, q, cache->page_table_stride);
    REQ(ws, MXS_EWORKSPACE, "index_score_topk: no scores buffer and no workspace");
    REQ(ws_bytes >= need, MXS_EWORKSPACE, "index_score_topk: workspace %zu bytes, needs %zu", ws_bytes, need);
    REQ(aligned(ws, 16), MXS_EINVAL, "ws: not 16-byte aligned");
    sc = static_cast<float *>(ws);
  }
  REQ(aligned(sc, 4), MXS_EINVAL, "scores: misaligned");
  if (B == 0) return ok();
  const mxs::CacheView c = view(cache);
  if (int r = launched(mxs::launch_index_score(c, q_idx, w, B, q, H_I, sc, mxs::StepStore{}, (hipStream_t)stream),
                       "index_score"))
    return r;
  return launched(mxs::launch_topk(c, sc, B, q, topk, block_table, (hipStream_t)stream), "topk_blocks");
}

int mxs_default_partitions(int32_t B, int32_t q_rows, int32_t topk) {
  return default_partitions(B, q_rows, topk);
}

int mxs_default_partitions_for(int32_t B, int32_t q_rows, int32_t topk, int32_t kv_format) {
  (void)kv_format;                                 // the same rule for every format
  return default_partitions(B, q_rows, topk);
}

static int check_attn_args(const mxs_cache *cache, const void *q, int32_t q_dtype, const int32_t *block_table,
                           int32_t B, int32_t q_rows, int32_t H, int32_t topk, int32_t P, float sm_scale) {
  if (int r = check_cache(cache, false, true)) return r;
  if (int r = check_rows(B, q_rows)) return r;
  if (int r = check_topk(topk)) return r;
  REQ(H >= 1, MXS_EINVAL, "H: %d, must be >= 1", H);
  REQ(H <= MXS_MAX_H, MXS_EUNSUPPORTED, "H: %d query heads per KV head, more than %d", H, MXS_MAX_H);
  REQ(P >= 1, MXS_EINVAL, "num_partitions: %d, must be >= 1", P);
  REQ(P <= MXS_MAX_PARTITIONS, MXS_EUNSUPPORTED, "num_partitions: %d, more than %d", P, MXS_MAX_PARTITIONS);
  REQ(std::isfinite(sm_scale), MXS_EINVAL, "sm_scale: not finite");
  if (cache->kv_format == MXS_FMT_MXFP4)
    REQ(q_dtype == MXS_E4M3, MXS_EUNSUPPORTED, "q_dtype: %d; an MXFP4 KV cache takes an e4m3 query", q_dtype);
  else
    REQ(q_dtype == MXS_BF16, MXS_EUNSUPPORTED, "q_dtype: %d; an FP8 or NVFP4 KV cache takes a bf16 query", q_dtype);
  REQ(q && aligned(q, 16), MXS_EINVAL, "q: null or not 16-byte aligned");
  REQ(block_table && aligned(block_table, 4), MXS_EINVAL, "block_table: null or misaligned");
  return MXS_OK;
}

int sparse_split_attn(const mxs_cache *cache, const void *q, int32_t q_dtype, const int32_t *block_table, int32_t B,
                      int32_t q_rows, int32_t H, int32_t topk, int32_t num_partitions, float sm_scale, float *sp_m,
                      float *sp_l, float *sp_o, void *stream) {
  REQ(cache, MXS_EINVAL, "cache: null");
  const int32_t P = num_partitions == 0 ? default_partitions(B, q_rows, topk) : num_partitions;
  if (int r = check_attn_args(cache, q, q_dtype, block_table, B, q_rows, H, topk, P, sm_scale)) return r;
  REQ(sp_m && sp_l && sp_o, MXS_EINVAL, "sp_m / sp_l / sp_o: null");
  REQ(aligned(sp_m, 4) && aligned(sp_l, 4) && aligned(sp_o, 16), MXS_EINVAL, "sp_m / sp_l / sp_o: misaligned");
  if (B == 0) return ok();
  return launched(mxs::launch_split_attn(view(cache), q, q_dtype, block_table, B, q_rows, H, topk, P, sm_scale, sp_m,
                                         sp_l, sp_o, (hipStream_t)stream),
                  "sparse_split_attn");
}

int lse_merge(const float *sp_m, const float *sp_l, const float *sp_o, int32_t n_rows, int32_t P, uint16_t *out,
              float *lse, void *stream) {
  REQ(n_rows >= 0, MXS_EINVAL, "n_rows: %d, must be >= 0", n_rows);
  REQ(P >= 1, MXS_EINVAL, "P: %d, must be >= 1", P);
  REQ(P <= MXS_MAX_PARTITIONS, MXS_EUNSUPPORTED, "P: %d, more than %d", P, MXS_MAX_PARTITIONS);
  if (n_rows == 0) return ok();
  REQ(sp_m && sp_l && sp_o && out, MXS_EINVAL, "sp_m / sp_l / sp_o / out: null");
  REQ(aligned(sp_o, 8) && aligned(out, 4) && aligned(sp_m, 4) && aligned(sp_l, 4), MXS_EINVAL,
      "lse_merge: misaligned buffer (sp_o 8 B, out 4 B)");
  REQ(!lse || aligned(lse, 4), MXS_EINVAL, "lse: misaligned");
  return launched(mxs::launch_lse_merge(sp_m, sp_l, sp_o, n_rows, P, out, lse, (hipStream_t)stream), "lse_merge");
}

int mxs_read_index_pages(const mxs_cache *cache, int32_t B, uint32_t *sink, void *stream) {
  if (int r = check_cache(cache, true, false)) return r;
  REQ(B >= 0, MXS_EINVAL, "B: %d, must be >= 0", B);
  REQ(sink && aligned(sink, 4), MXS_EINVAL, "sink: null or misaligned");
  if (B == 0) return ok();
  return launched(mxs::launch_read_pages(view(cache), B, (uint32_t)page_bytes(cache->idx_format), sink,
                                         (hipStream_t)stream),
                  "mxs_read_index_pages");
}

size_t mxs_workspace_bytes(int32_t B, int32_t q, int32_t H, int32_t H_I, int32_t topk, int32_t page_table_stride,
                           int32_t num_partitions) {
  (void)H_I;
  if (B < 0 || q < 0 || H < 0 || topk < 0 || page_table_stride < 0) return 0;
  const int32_t P = num_partitions == 0 ? default_partitions(B, q, topk) : num_partitions;
  return step_ws(B, q, H, topk, page_table_stride, P).total;
}

int mxs_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  REQ(ws || ws_bytes == 0, MXS_EINVAL, "mxs_workspace_init: ws null");
  REQ(aligned(ws, 256), MXS_EINVAL, "mxs_workspace_init: ws not 256-byte aligned");
  REQ(ws_bytes % 4 == 0, MXS_EINVAL, "mxs_workspace_init: ws_bytes %zu not a multiple of 4", ws_bytes);
  if (ws_bytes == 0) return ok();
  return launched(mxs::launch_zero(static_cast<uint32_t *>(ws), ws_bytes / 4, (hipStream_t)stream),
                  "mxs_workspace_init");
}

// The argument checks of decode_step (and of decode_step_one_launch), then
// the launches of the one or the other.
static int step_entry(const mxs_step *a, void *ws, size_t ws_bytes, void *stream, bool one_launch) {
  REQ(a, MXS_EINVAL, "step: null");
  const mxs_cache *cache = &a->cache;
  if (int r = check_cache(cache, true, true)) return r;
  if (int r = check_rows(a->B, a->q)) return r;
  if (int r = check_topk(a->topk)) return r;
  if (a->B == 0) return ok();                      // an empty batch: nothing to do
  const int32_t P =
      a->num_partitions == 0 ? default_partitions(a->B, a->q, a->topk) : a->num_partitions;
  const bool mx = cache->kv_format == MXS_FMT_MXFP4;
  if (mx)
    REQ(a->q_dtype == MXS_F32 || a->q_dtype == MXS_BF16, MXS_EUNSUPPORTED,
        "q_dtype: %d; an MXFP4 KV step takes an fp32 or bf16 query and stores it as e4m3", a->q_dtype);
  else
    REQ(a->q_dtype == MXS_BF16, MXS_EUNSUPPORTED, "q_dtype: %d; an FP8 or NVFP4 KV step takes a bf16 query",
        a->q_dtype);
  REQ(a->query && aligned(a->query, 16), MXS_EINVAL, "query: null or not 16-byte aligned");
  const bool store = a->k_new || a->v_new || a->idx_new;
  if (store)
    REQ(a->k_new && a->v_new && a->idx_new && aligned(a->k_new, 8) && aligned(a->v_new, 8) && aligned(a->idx_new, 8),
        MXS_EINVAL, "k_new / v_new / idx_new: give all three (8-byte aligned) or none");
  if (int r = check_score_args(cache, a->q_idx, a->w, a->B, a->q, a->H_I)) return r;
  REQ(a->H >= 1, MXS_EINVAL, "H: %d, must be >= 1", a->H);
  REQ(a->H <= MXS_MAX_H, MXS_EUNSUPPORTED, "H: %d query heads per KV head, more than %d", a->H, MXS_MAX_H);
  REQ(P >= 1 && P <= MXS_MAX_PARTITIONS, MXS_EUNSUPPORTED, "num_partitions: %d, must be in 1..%d", P,
      MXS_MAX_PARTITIONS);
  REQ(std::isfinite(a->sm_scale), MXS_EINVAL, "sm_scale: not finite");
  REQ(a->out && aligned(a->out, 4), MXS_EINVAL, "out: null or misaligned");
  REQ(!a->lse || aligned(a->lse, 4), MXS_EINVAL, "lse: misaligned");
  REQ(!a->block_table_out || aligned(a->block_table_out, 4), MXS_EINVAL, "block_table_out: misaligned");
  REQ(!a->scores_out || aligned(a->scores_out, 4), MXS_EINVAL, "scores_out: misaligned");
  const StepWs w = step_ws(a->B, a->q, a->H, a->topk, cache->page_table_stride, P);
  REQ(ws, MXS_EWORKSPACE, "decode_step: workspace null (needs %zu bytes)", w.total);
  REQ(ws_bytes >= w.total, MXS_EWORKSPACE, "decode_step: workspace %zu bytes, needs %zu", ws_bytes, w.total);
  REQ(aligned(ws, 256), MXS_EINVAL, "ws: not 256-byte aligned");

  uint8_t *base = static_cast<uint8_t *>(ws);
  float *scores = a->scores_out ? a->scores_out : reinterpret_cast<float *>(base + w.scores);
  int32_t *table = a->block_table_out ? a->block_table_out : reinterpret_cast<int32_t *>(base + w.table);
  uint8_t *q8 = base + w.q8;
  float *sp_m = reinterpret_cast<float *>(base + w.sp_m);
  float *sp_l = reinterpret_cast<float *>(base + w.sp_l);
  float *sp_o = reinterpret_cast<float *>(base + w.sp_o);
  uint64_t *counters = reinterpret_cast<uint64_t *>(base + w.counters);
  uint32_t *seq_cnt = reinterpret_cast<uint32_t *>(base + w.seq_cnt);
  const hipStream_t s = (hipStream_t)stream;
  const mxs::CacheView c = view(cache);
  const void *qa = mx ? static_cast<const void *>(q8) : a->query;
  mxs::FusedMerge fm;
  fm.counters = counters;
  fm.out = a->out;
  fm.lse = a->lse;

  if (one_launch) {
    // the whole step as one launch: scoring workgroups (with the row and query
    // stores, device-coherent), then attention workgroups that wait for their
    // sequence; the merge counters and sequence counters reset themselves
    REQ(mxs::decode_step_one_launch(c, a->B, a->q), MXS_EUNSUPPORTED,
        "decode_step_one_launch: needs MXFP4 K / V and index caches, q <= 8 and B x page_table_stride >= 8192 "
        "(got formats %d / %d, q = %d, %lld pages)", cache->kv_format, cache->idx_format, a->q,
        (long long)a->B * cache->page_table_stride);
    mxs::StepStore st;
    if (store) {
      st.k_new = a->k_new;
      st.v_new = a->v_new;
      st.idx_new = a->idx_new;
    }
    st.q_att = a->query;
    st.q_dtype = a->q_dtype;
    st.H = a->H;
    st.q8 = q8;
    return launched(mxs::launch_decode_step(c, a->q_idx, a->w, a->B, a->q, a->H_I, scores, st, a->H, a->topk, P,
                                            a->sm_scale, table, sp_m, sp_l, sp_o, fm, seq_cnt, s),
                    "decode_step_one_launch");
  }

  // 1 - 3: the new rows into the pages, q -> e4m3 and the scores, one launch
  // (the waves that own a page holding new positions store those index rows
  // before scoring it; K / V rows and q are read only by the attention
  // launch); it also clears the attention launch's per-row merge counters
  mxs::StepStore st;
  st.counters = counters;
  if (store) {
    st.k_new = a->k_new;
    st.v_new = a->v_new;
    st.idx_new = a->idx_new;
  }
  if (mx) {
    st.q_att = a->query;
    st.q_dtype = a->q_dtype;
    st.H = a->H;
    st.q8 = q8;
  }
  if (int r = launched(mxs::launch_index_score(c, a->q_idx, a->w, a->B, a->q, a->H_I, scores, st, s),
                       "decode_step: store + score"))
    return r;
  // 4 - 6: top-k, split attention and merge, one launch: every attention
  // workgroup selects its row's blocks from the scores itself (partition 0
  // writes the row's block table), and the row's last partition to finish
  // merges the row
  return launched(mxs::launch_select_attn(c, scores, qa, a->B, a->q, a->H, a->topk, P, a->sm_scale, table, sp_m, sp_l,
                                          sp_o, fm, s),
                  "decode_step: top-k + split attention + merge");
}

int decode_step(const mxs_step *a, void *ws, size_t ws_bytes, void *stream) {
  return step_entry(a, ws, ws_bytes, stream, false);
}

int decode_step_one_launch(const mxs_step *a, void *ws, size_t ws_bytes, void *stream) {
  return step_entry(a, ws, ws_bytes, stream, true);
}

// The argument checks of decode_step_reuse (and of decode_step_reuse_one_launch),
// then the launches of the one or the other.
static int reuse_entry(const mxs_step *a, const int32_t *block_table, void *ws, size_t ws_bytes, void *stream,
                       bool one_launch) {
  const char *name = one_launch ? "decode_step_reuse_one_launch" : "decode_step_reuse";
  REQ(a, MXS_EINVAL, "step: null");
  const mxs_cache *cache = &a->cache;
  if (int r = check_cache(cache, false, true)) return r;
  if (int r = check_rows(a->B, a->q)) return r;
  if (int r = check_topk(a->topk)) return r;
  if (a->B == 0) return ok();                      // an empty batch: nothing to do
  const int32_t P =
      a->num_partitions == 0 ? default_partitions(a->B, a->q, a->topk) : a->num_partitions;
  const bool mx = cache->kv_format == MXS_FMT_MXFP4;
  if (mx)
    REQ(a->q_dtype == MXS_F32 || a->q_dtype == MXS_BF16, MXS_EUNSUPPORTED,
        "q_dtype: %d; an MXFP4 KV step takes an fp32 or bf16 query and stores it as e4m3", a->q_dtype);
  else
    REQ(a->q_dtype == MXS_BF16, MXS_EUNSUPPORTED, "q_dtype: %d; an FP8 or NVFP4 KV step takes a bf16 query",
        a->q_dtype);
  REQ(a->query && aligned(a->query, 16), MXS_EINVAL, "query: null or not 16-byte aligned");
  REQ(!a->k_new == !a->v_new, MXS_EINVAL, "k_new / v_new: give both or neither");
  REQ((!a->k_new || aligned(a->k_new, 8)) && (!a->v_new || aligned(a->v_new, 8)), MXS_EINVAL,
      "k_new / v_new: not 8-byte aligned");
  REQ(block_table && aligned(block_table, 4), MXS_EINVAL, "block_table: null or misaligned");
  REQ(a->H >= 1, MXS_EINVAL, "H: %d, must be >= 1", a->H);
  REQ(a->H <= MXS_MAX_H, MXS_EUNSUPPORTED, "H: %d query heads per KV head, more than %d", a->H, MXS_MAX_H);
  REQ(P >= 1 && P <= MXS_MAX_PARTITIONS, MXS_EUNSUPPORTED, "num_partitions: %d, must be in 1..%d", P,
      MXS_MAX_PARTITIONS);
  REQ(std::isfinite(a->sm_scale), MXS_EINVAL, "sm_scale: not finite");
  REQ(a->out && aligned(a->out, 4), MXS_EINVAL, "out: null or misaligned");
  REQ(!a->lse || aligned(a->lse, 4), MXS_EINVAL, "lse: misaligned");
  const StepWs w = step_ws(a->B, a->q, a->H, a->topk, cache->page_table_stride, P);
  REQ(ws, MXS_EWORKSPACE, "%s: workspace null (needs %zu bytes)", name, w.total);
  REQ(ws_bytes >= w.total, MXS_EWORKSPACE, "%s: workspace %zu bytes, needs %zu", name, ws_bytes, w.total);
  REQ(aligned(ws, 256), MXS_EINVAL, "ws: not 256-byte aligned");

  uint8_t *base = static_cast<uint8_t *>(ws);
  uint8_t *q8 = base + w.q8;
  float *sp_m = reinterpret_cast<float *>(base + w.sp_m);
  float *sp_l = reinterpret_cast<float *>(base + w.sp_l);
  float *sp_o = reinterpret_cast<float *>(base + w.sp_o);
  uint64_t *counters = reinterpret_cast<uint64_t *>(base + w.counters);
  uint32_t *seq_cnt = reinterpret_cast<uint32_t *>(base + w.seq_cnt);
  const hipStream_t s = (hipStream_t)stream;
  const mxs::CacheView c = view(cache);
  mxs::FusedMerge fm;
  fm.counters = counters;
  fm.out = a->out;
  fm.lse = a->lse;

  if (one_launch)   // store workgroups, then attention workgroups that wait for their sequence's stores
    return launched(mxs::launch_reuse_step(c, a->k_new, a->v_new, a->query, a->q_dtype, block_table, a->B, a->q,
                                           a->H, a->topk, P, a->sm_scale, sp_m, sp_l, sp_o, fm, seq_cnt, s),
                    name);

  // 1 - 2: the new K / V rows into the pages, q -> e4m3 (MXFP4 KV) and the
  // merge counters cleared, one launch
  if (int r = launched(mxs::launch_reuse_store(c, a->k_new, a->v_new, a->query, a->q_dtype, a->H, mx ? q8 : nullptr,
                                               counters, a->B, a->q, s),
                       "decode_step_reuse: store"))
    return r;
  // 5 - 6: split attention over the given blocks and the merge, one launch
  const void *qa = mx ? static_cast<const void *>(q8) : a->query;
  return launched(mxs::launch_table_attn(c, block_table, qa, a->B, a->q, a->H, a->topk, P, a->sm_scale, sp_m, sp_l,
                                         sp_o, fm, s),
                  "decode_step_reuse: split attention + merge");
}

int decode_step_reuse(const mxs_step *a, const int32_t *block_table, void *ws, size_t ws_bytes, void *stream) {
  return reuse_entry(a, block_table, ws, ws_bytes, stream, false);
}

int decode_step_reuse_one_launch(const mxs_step *a, const int32_t *block_table, void *ws, size_t ws_bytes,
                                 void *stream) {
  return reuse_entry(a, block_table, ws, ws_bytes, stream, true);
}

}  // extern "C"
