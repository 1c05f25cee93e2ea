/*
 * mxsparse — one tensor-parallel rank's sparse-attention decode step over
 * MXFP4 (or FP8, or NVFP4) paged caches, for AMD MI355X (gfx950).
 *
 * The step (ATOM PR #2812, "[MiniMax-M3.1] Mono decode over the MXFP4 KV and
 * index caches": What, and its commit messages):
 *   1. row store   new index-key, K and V rows are quantized into 128-token
 *                  cache pages (MXFP4: 32-element e2m1 groups with e8m0 scales,
 *                  8704 bytes per page at head_dim 128);
 *   2. q store     the attention query is packed to saturating e4m3;
 *   3. index score every page of the index cache is scored against the step's
 *                  query rows;
 *   4. top-k       each query row keeps its k best blocks (one block = one page);
 *   5. split attn  softmax attention over the selected pages only, written as
 *                  per-partition partials (sp_m, sp_l, sp_o);
 *   6. merge       the partials are combined by log-sum-exp.
 *
 * Conventions, for every entry point:
 *   - Pointers named in a struct or argument list are DEVICE pointers unless the
 *     comment says "host". They are owned by the caller; the library allocates
 *     and frees nothing and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is only enqueued:
 *     no host synchronization, no device-to-host read, so every call may be
 *     captured into a HIP graph.
 *   - Arguments are validated on the host before anything is enqueued; an error
 *     return means nothing was launched. mxs_last_error() then names the
 *     offending argument (thread-local string, valid until the next call).
 *   - Values that live in device memory (page ids, slots, context lengths,
 *     block ids) cannot be checked on the host. Kernels skip out-of-range page
 *     ids and slots (nothing is read or written through them) and treat
 *     out-of-range block ids as empty. Device faults surface at the caller's
 *     next synchronization.
 *   - MXS_ELAUNCH reports a launch failure (hipGetLastError after enqueue).
 *
 * Cache page layouts (a reading: the scorer of the same PR reads a tile with one
 * 16-byte load of key codes and one dword of e8m0 scales, commit message of the
 * MXFP4 index-cache commit; one layout serves the index keys, K and V, commit
 * message of the MXFP4 main-KV commit):
 *   MXFP4 page, 8704 B: token t (0..127) has its 128 e2m1 codes at bytes
 *     [64 t, 64 t + 64) — element 2i in the low nibble of byte i, 2i+1 in the
 *     high nibble — and its four e8m0 group scales (elements 0-31, 32-63, 64-95,
 *     96-127) at bytes 8192 + 4 t + g.
 *   FP8 page, 16896 B: token t has its 128 e4m3 codes at [128 t, 128 t + 128)
 *     and its fp32 scale at 16384 + 4 t (value = e4m3(code) * scale).
 *   NVFP4 page, 9728 B: token t has its codes at [64 t, 64 t + 64) as in the
 *     MXFP4 page, the e4m3 scale codes of its eight 16-element blocks at
 *     8192 + 8 t + b and its fp32 scale at 9216 + 4 t (value = e2m1(code) *
 *     e4m3(block code) * scale). The pages name NVFP4 K/V and index caches
 *     (ATOM PR #2686, timeline entry #2744; ATOM PR #2812, commit messages)
 *     without defining them: this is the public NVFP4 layout (e2m1 in
 *     16-element blocks, e4m3 block scales, a second-level fp32 scale) with the
 *     second level kept per token, a reading.
 * Slot s of a pool is token s % 128 of page s / 128.
 *
 * Shapes: head_dim 128 everywhere; one KV head shared by H query heads (GQA);
 * B sequences with q query rows each (1 + speculative drafts); query row j of
 * sequence b sits at position L_b - q + j, where L_b (context_lens[b]) already
 * counts the step's q new rows, and sees positions <= its own (causal).
 */
#ifndef MXSPARSE_H
#define MXSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXS_ABI_VERSION 1

typedef enum {
    MXS_OK = 0,
    MXS_EINVAL = 1,          /* a null pointer, a bad size, misalignment            */
    MXS_EUNSUPPORTED = 2,    /* a shape or format this library refuses (see below)  */
    MXS_EWORKSPACE = 3,      /* workspace missing or smaller than required           */
    MXS_ELAUNCH = 4          /* the HIP runtime rejected a launch                     */
} mxs_status;

typedef enum { MXS_FMT_MXFP4 = 0, MXS_FMT_FP8 = 1, MXS_FMT_NVFP4 = 2 } mxs_format;
typedef enum { MXS_F32 = 0, MXS_BF16 = 1, MXS_E4M3 = 2 } mxs_dtype;

#define MXS_PAGE_TOKENS 128
#define MXS_HEAD_DIM 128
#define MXS_MXFP4_PAGE_BYTES 8704
#define MXS_FP8_PAGE_BYTES 16896
#define MXS_NVFP4_PAGE_BYTES 9728

/* Refusal limits (MXS_EUNSUPPORTED): H <= 16 query heads per KV head,
 * 1 <= H_I <= 4 index heads, q <= 16 query rows per sequence, topk <= 64,
 * page_table_stride <= 8192 pages (1M tokens), partitions <= 64.
 * Format ids other than MXS_FMT_MXFP4, MXS_FMT_FP8 and MXS_FMT_NVFP4 are
 * refused. */
#define MXS_MAX_H 16
#define MXS_MAX_H_I 4
#define MXS_MAX_Q 16
#define MXS_MAX_TOPK 64
#define MXS_MAX_PAGES_PER_SEQ 8192
#define MXS_MAX_PARTITIONS 64

/* The paged caches of one layer. The struct itself is host memory. */
typedef struct {
    uint8_t *k_pages;              /* [num_pages][page bytes of kv_format], 16 B aligned   */
    uint8_t *v_pages;              /* same layout as k_pages                               */
    uint8_t *idx_pages;            /* [num_pages][page bytes of idx_format], 16 B aligned  */
    int32_t num_pages;             /* pool size in pages; page ids must be < num_pages     */
    int32_t kv_format;             /* mxs_format of k_pages / v_pages                      */
    int32_t idx_format;            /* mxs_format of idx_pages                              */
    const int32_t *page_table;     /* [B][page_table_stride] physical page of each logical
                                      page; the same ids index all three pools            */
    int32_t page_table_stride;     /* logical pages per sequence row (>= max ceil(L/128))  */
    const int32_t *context_lens;   /* [B] L_b, including the step's q new rows; 1 <= L_b  */
} mxs_cache;

/* ---- 1. row store --------------------------------------------------------
 * mxfp4_row_store: quantize n fp32 rows of 128 into MXFP4 slots (same PR,
 * commit messages of the MXFP4 index-cache and main-KV commits). Per 32-element
 * group: e8m0 scale byte = max(E(amax) - 2, 0), E(amax) being the biased fp32
 * exponent of the group's largest magnitude (the OCP MX v1.0 rule,
 * 2^(floor(log2 amax) - 2)); each element divided by the scale and rounded to
 * e2m1 (nearest, ties to even, |v| > 6 saturates to 6, sign kept so a small
 * negative value stores -0).
 *   rows  [n][128] fp32, 8 B aligned; finite values (non-finite input is outside
 *         the contract)
 *   slots [n] int64: page * 128 + token; a slot < 0 or >= num_pages * 128 is
 *         skipped
 *   pages the MXFP4 pool [num_pages][8704], 16 B aligned
 * fp8_row_store: the same for an FP8 pool: per token scale = fp32(amax / 448)
 * (1 for an all-zero row), codes = saturating e4m3 of fp32(x / scale). The
 * pages give an FP8 cache with a per-token fp32 scale but no rule (ATOM PR
 * #2686, "Enable Mono decode with fixed DSpark verify", Summary); this rule is
 * a reading.
 * nvfp4_row_store: the same for an NVFP4 pool [num_pages][9728] (a reading, see
 * the page layouts above): per token S = fp32(amax / 2688) (2688 = 6 * 448; 1
 * for an all-zero row, 2^-149 where the quotient underflows to 0); per
 * 16-element block c_b = saturating e4m3 of fp32(a_b / fp32(6 S)), a_b the
 * block's largest magnitude; each element e2m1 of fp32(x / fp32(e4m3(c_b) S)),
 * code 0 where that divisor is 0. */
int mxfp4_row_store(const float *rows, int64_t n, const int64_t *slots, uint8_t *pages,
                    int32_t num_pages, void *stream);
int fp8_row_store(const float *rows, int64_t n, const int64_t *slots, uint8_t *pages,
                  int32_t num_pages, void *stream);
int nvfp4_row_store(const float *rows, int64_t n, const int64_t *slots, uint8_t *pages,
                    int32_t num_pages, void *stream);

/* ---- 2. q store ----------------------------------------------------------
 * pack_q_e4m3: n elements of q (fp32 or bf16 per q_dtype) to OCP e4m3 codes
 * with unit scale: round to nearest even, |x| > 448 and +-inf saturate to
 * +-448, NaN stays NaN (0x7F with the sign bit kept) (same PR, commit messages
 * of the e4m3 q store and of pack_q_e4m3). q: 4 B (fp32) or 2 B (bf16)
 * aligned; q8: [n] bytes. */
int pack_q_e4m3(const void *q, int32_t q_dtype, int64_t n, uint8_t *q8, void *stream);

/* ---- 3. index score ------------------------------------------------------
 * index_score: block scores of every candidate block of every query row
 * (the block score of the tiny decode configuration, read by the index scorer
 * of the MXFP4 index-cache commit):
 *   S[b][j][i] = max over tokens t of block i with t <= pos_j of
 *                sum_h w[b][j][h] * max(0, q_idx[b][j][h] . k_idx[t])
 * Block i is a candidate of row j when 128 i <= pos_j; entries of other blocks
 * below page_table_stride are written as -inf.
 *   q_idx  [B][q][H_I][128] bf16 bits, 16 B aligned
 *   w      [B][q][H_I] fp32
 *   scores [B][q][page_table_stride] fp32 (output) */
int index_score(const mxs_cache *cache, const uint16_t *q_idx, const float *w, int32_t B,
                int32_t q, int32_t H_I, float *scores, void *stream);

/* ---- 4. top-k ------------------------------------------------------------
 * topk_blocks: per query row, the topk highest-scoring candidate blocks; ties
 * go to the lower block id; a row with fewer than topk candidates keeps all of
 * them. Output ids are ascending, padded with -1.
 *   scores      [B][q][page_table_stride] fp32 as written by index_score
 *   block_table [B][q][topk] int32 (output) */
int topk_blocks(const mxs_cache *cache, const float *scores, int32_t B, int32_t q, int32_t topk,
                int32_t *block_table, void *stream);

/* index_score_topk: index_score then topk_blocks, with the scores in the
 * workspace (ws_bytes >= mxs_score_workspace_bytes(B, q, page_table_stride)),
 * or in `scores` when it is non-null (then ws may be null). */
int index_score_topk(const mxs_cache *cache, const uint16_t *q_idx, const float *w, int32_t B,
                     int32_t q, int32_t H_I, int32_t topk, int32_t *block_table, float *scores,
                     void *ws, size_t ws_bytes, void *stream);
size_t mxs_score_workspace_bytes(int32_t B, int32_t q, int32_t page_table_stride);

/* ---- 5. split attention --------------------------------------------------
 * sparse_split_attn: for each query row (b, j), head h and partition p, the
 * unnormalized softmax partial over the tokens t <= pos_j of the blocks in
 * block-table slots [p c, min((p + 1) c, topk)), c = ceil(topk / P):
 *   s_t = sm_scale * q[b][j][h] . K[t];  m = max s;  l = sum exp(s - m);
 *   o = sum exp(s_t - m) V[t]
 * A partition without tokens writes (m, l, o) = (-inf, 0, 0) (same PR, commit
 * message of the MXFP4 main-KV commit: split stage, sp_o / sp_m / sp_l).
 *   q     MXFP4 KV: e4m3 codes (q_dtype MXS_E4M3) [B][q][H][128];
 *         FP8 or NVFP4 KV: bf16 bits (q_dtype MXS_BF16) [B][q][H][128]; 16 B aligned
 *   block_table [B][q][topk] int32 block ids (-1 = empty slot)
 *   sp_m, sp_l  [B][q][H][P] fp32;  sp_o [B][q][H][P][128] fp32 (outputs)
 * P = num_partitions in 1..64 (0: mxs_default_partitions_for(B, q_rows, topk,
 * cache->kv_format)). */
int sparse_split_attn(const mxs_cache *cache, const void *q, int32_t q_dtype,
                      const int32_t *block_table, int32_t B, int32_t q_rows, int32_t H,
                      int32_t topk, int32_t num_partitions, float sm_scale, float *sp_m,
                      float *sp_l, float *sp_o, void *stream);
/* The partition count the library takes for num_partitions = 0, the same
 * for every K / V format: P = min(ceil(topk / 4), cap) with cap = max(1, 256 /
 * (B q_rows)) — one block per wave of a 4-wave workgroup, but no more
 * workgroups than MI355X has CUs once the rows alone fill it; if P B q_rows
 * is then below 256, min(ceil(topk / 2), cap) instead (two blocks per
 * workgroup, which its waves take as half blocks); clamped to 1..64. A
 * choice of this library; the pages fix none. kv_format is not consulted
 * (kept so that callers can state the format).
 * mxs_default_partitions: the same. */
int mxs_default_partitions_for(int32_t B, int32_t q_rows, int32_t topk, int32_t kv_format);
int mxs_default_partitions(int32_t B, int32_t q_rows, int32_t topk);

/* ---- 6. merge ------------------------------------------------------------
 * lse_merge: M = max_p m_p; L = sum_p l_p exp(m_p - M); O = sum_p o_p
 * exp(m_p - M) / L; lse = M + ln L. Empty partitions weigh nothing; a row with
 * only empty partitions gives O = 0, lse = -inf.
 *   sp_m, sp_l [n_rows][P]; sp_o [n_rows][P][128] fp32
 *   out [n_rows][128] bf16 bits (round to nearest even); lse [n_rows] fp32 or null */
int lse_merge(const float *sp_m, const float *sp_l, const float *sp_o, int32_t n_rows, int32_t P,
              uint16_t *out, float *lse, void *stream);

/* ---- the whole step ------------------------------------------------------ */
typedef struct {
    mxs_cache cache;
    const float *k_new;        /* [B][q][128] fp32 rows for positions L_b - q + j; null = */
    const float *v_new;        /*   the cache already holds them (no row store)           */
    const float *idx_new;
    const void *query;         /* attention query [B][q][H][128]: MXFP4 KV takes fp32 or
                                  bf16 (q_dtype) and stores it as e4m3; FP8 and NVFP4
                                  KV take bf16                                          */
    int32_t q_dtype;
    const uint16_t *q_idx;     /* [B][q][H_I][128] bf16 bits                            */
    const float *w;            /* [B][q][H_I] fp32                                      */
    int32_t B, q, H, H_I, topk, num_partitions;   /* num_partitions 0 = default          */
    float sm_scale;
    uint16_t *out;             /* [B][q][H][128] bf16 bits (output)                     */
    float *lse;                /* [B][q][H] fp32 or null                                */
    int32_t *block_table_out;  /* [B][q][topk] int32 or null: the step's selection      */
    float *scores_out;         /* [B][q][page_table_stride] fp32 or null                */
} mxs_step;

/* decode_step: the six stages above on one stream, as two launches: the index
 * scores (which also store the step's new K / V / index rows and its e4m3
 * query), then top-k, split attention and the log-sum-exp merge (each row's
 * last partition workgroup merges the row). ws: device workspace of at least
 * mxs_workspace_bytes(...) bytes, 256 B aligned; its contents need no
 * initialization and are scratch after the call (it holds the per-row merge
 * counters, cleared by the first launch), so two calls in flight at once must
 * not share one. mxs_workspace_bytes with num_partitions = 0 sizes for the
 * default partition count (mxs_default_partitions), which is the same for
 * every cache format. */
int decode_step(const mxs_step *step, void *ws, size_t ws_bytes, void *stream);
size_t mxs_workspace_bytes(int32_t B, int32_t q, int32_t H, int32_t H_I, int32_t topk,
                           int32_t page_table_stride, int32_t num_partitions);

/* decode_step_one_launch: the same step, results bit for bit those of
 * decode_step, as ONE launch (the single-launch step of the pages' persistent
 * decode kernel, vLLM PR #60528, Merge Danger, which assumes every workgroup
 * co-resident). The grid holds the scoring workgroups first, then the
 * attention workgroups. A scoring workgroup writes its scores, its share of
 * the step's K / V rows and of the e4m3 query with device-coherent stores and
 * counts itself in for its sequence; an attention workgroup waits for its
 * sequence's count, then selects, attends and merges. An attention workgroup
 * only waits for workgroups with lower ids, which in-order dispatch has
 * already started and which wait for nothing, so no co-residency is assumed;
 * the wait is also bounded (about a second), so a launch always ends.
 *   Supported: MXFP4 K / V and index caches, q <= 8 query rows and
 *   B x page_table_stride >= 8192 pages (else MXS_EUNSUPPORTED, nothing
 *   launched).
 *   ws: as for decode_step, but zero-filled before its first use
 *   (mxs_workspace_init, or a zero-filled allocation): it also holds
 *   per-sequence counters, and every call leaves them zero again, so one
 *   workspace serves any number of calls in stream order.
 *   Measured on MI355X (4 x 8 rows, 256K context): slower than decode_step
 *   (44 us against 36 us per step): its attention workgroups need the whole
 *   register file of a CU, so none can start until a scoring workgroup has
 *   left its CU, and the scan inside the larger kernel runs slower (22.7 us
 *   against 19.2 us alone). */
int decode_step_one_launch(const mxs_step *step, void *ws, size_t ws_bytes, void *stream);
/* mxs_workspace_init: zero-fill ws_bytes (a multiple of 4) of a workspace on
 * `stream` (a kernel, not a memset, so it may be captured in a HIP graph).
 * Errors: MXS_EINVAL for a null or misaligned ws; MXS_ELAUNCH. */
int mxs_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* decode_step_reuse: the step of a layer that reuses an earlier layer's sparse
 * block selection instead of making its own (ATOM PR #2686, "Enable Mono
 * decode with fixed DSpark verify": under an index_topk_freq schedule some
 * sparse layers reuse a selection; the first layer still selects its own).
 * Stages 1, 2, 5 and 6 on one stream, as two launches: the step's new K and
 * V rows into the pages and the query as e4m3 (MXFP4 KV), then split
 * attention over the given blocks and the merge. Nothing of the index side
 * is read or written: step->idx_new, q_idx, w, H_I, block_table_out and
 * scores_out and cache.idx_pages are ignored; k_new and v_new are given both
 * or neither.
 *   block_table  [B][q][topk] int32: the reused selection (as topk_blocks
 *                writes it: ascending, -1 padded); entries < 0, >= the page
 *                table stride or past the row's position are skipped
 *   ws           as for decode_step (mxs_workspace_bytes, 256 B aligned,
 *                scratch; calls in flight at once must not share one)
 * Errors as for decode_step; MXS_EINVAL when block_table is null. */
int decode_step_reuse(const mxs_step *step, const int32_t *block_table, void *ws, size_t ws_bytes,
                      void *stream);

/* decode_step_reuse_one_launch: decode_step_reuse as one launch (the same
 * step as above, ATOM PR #2686). The grid holds one store workgroup per
 * query row (its new K and V rows, device-coherent stores), then the
 * attention workgroups of decode_step_reuse. With an MXFP4 KV cache each of
 * them rounds the query to e4m3 in registers (the same codes pack_q_e4m3
 * stores), and a wave whose token range holds one of the step's new positions
 * waits (a bounded spin) until every store workgroup of its sequence has
 * counted in, just before it requests those pages; the other waves never
 * wait. Store workgroups have the lower ids and wait for nothing, and
 * workgroups are dispatched in increasing id order, so no wait depends on a
 * workgroup that cannot start. Output, lse and pages are bit for bit those of
 * decode_step_reuse.
 *   ws  as for decode_step_reuse, and zero before its first use
 *       (mxs_workspace_init): its merge counters and two counter words per
 *       sequence must start at zero; every call leaves them zero again (as
 *       do decode_step, decode_step_reuse and decode_step_one_launch on the
 *       same workspace), so a workspace is initialized once.
 * Arguments and errors as for decode_step_reuse. */
int decode_step_reuse_one_launch(const mxs_step *step, const int32_t *block_table, void *ws, size_t ws_bytes,
                                 void *stream);

/* decode_step_noalloc: decode_step for callers that cannot allocate device
 * memory (code under HIP graph capture that may not allocate, tight serving
 * loops, harnesses that forbid allocation). Same arguments, results, errors
 * and launches as decode_step, but the workspace is a device array the
 * library holds: MXS_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on, kept
 * until the process ends, zero when the library is loaded (every call leaves
 * its counter words zero again). Its device address is looked up once per
 * device (the calling thread's current device, which `stream` must belong to).
 * Nothing is allocated or freed by the call.
 *   Errors: MXS_EWORKSPACE when the step needs more workspace than the array
 *   holds (mxs_workspace_bytes(...) > MXS_NOALLOC_SCRATCH_BYTES: e.g. 4
 *   sequences x 8 rows at 256K context need about 2.4 MB, 32 x 8 about 4.6 MB);
 *   MXS_ELAUNCH when there is no usable current device; otherwise as
 *   decode_step.
 *   Concurrency: every call on one GPU shares that GPU's array (its contents
 *   from an earlier call, counters back at zero, do not matter); calls that
 *   overlap on one GPU — two streams, two threads — race on it and must be
 *   serialized by the caller. */
#define MXS_NOALLOC_SCRATCH_BYTES (8u << 20)
int decode_step_noalloc(const mxs_step *step, void *stream);

/* ---- diagnostics ---------------------------------------------------------- */

/* mxs_read_index_pages: a measurement aid, not a step of the method. It reads
 * every index page of sequences 0..B-1 once (logical pages 0..ceil(L_b/128)-1
 * through the page table, in page-table order, cache.idx_format's page size)
 * with plain 16-byte loads and nothing else, so its time is the streaming-read
 * ceiling of the scan that index_score performs (one workgroup per 4 logical
 * pages of a sequence, 256 threads, every load requested before any is used).
 * Page-table entries outside [0, num_pages) are not read.
 *   sink   device, >= 4 bytes, 4-byte aligned: may receive one word, whose
 *          value carries no meaning (it keeps the loads from being dropped)
 * Errors: MXS_EINVAL / MXS_EUNSUPPORTED for the cache as index_score checks
 * it (idx side only), B < 0 or a null / misaligned sink; MXS_ELAUNCH. */
int mxs_read_index_pages(const mxs_cache *cache, int32_t B, uint32_t *sink, void *stream);

const char *mxs_status_str(int status);
const char *mxs_last_error(void);
int mxs_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MXSPARSE_H */
