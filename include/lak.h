/*
 * lak.h -- C ABI of the layer-aware KV decode-attention library (gfx950 / MI355X).
 *
 * The method: "DELTA: Dynamic Layer-Aware Token Attention for Efficient
 * Long-Context Reasoning" (AI summary page, "Methodology in Plain English" and
 * "Main Findings").  A model's layers are split into three tiers that share one
 * paged KV cache kept whole in HBM (DELTA never evicts tokens):
 *   - full layers (the first two) attend to the whole context;
 *   - delta-layers also attend to the whole context and, from those softmax
 *     weights, score each token by its largest weight over the heads, score each
 *     page by adding its tokens' scores, and choose pages: a window of the newest
 *     pages plus, up to the budget, the older pages with the largest scores;
 *   - sparse layers attend to the tokens of the most recent choice only.
 *
 * Conventions shared by every entry point
 *   - Pointers named "device" point to HIP device memory owned by the caller; the
 *     library never allocates or frees device memory (its only device memory of its
 *     own is the static scratch of lak_attn_sparse_noalloc).  Pointers named "host"
 *     are ordinary host memory, read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call validates
 *     its arguments on the host, enqueues its kernels on `stream` and returns
 *     without synchronising.  On a negative status nothing was enqueued and
 *     lak_last_error() describes the reason.  Faults of kernels already enqueued
 *     surface as LAK_EHIP from a later call.
 *   - Shapes: B = active batch (set by lak_seq_reset), Hq query heads, Hkv KV
 *     heads, G = Hq / Hkv, D head dim, P page size.  Query head h reads KV head
 *     floor(h / G).  q / out are [B][Hq][D] row-major in the cache dtype; lse is
 *     [B][Hq] float32 (natural-log log-sum-exp of the scaled logits).
 *   - T_b (the current length of sequence b) always includes the token appended
 *     in the current decode step; NP_b = ceil(T_b / P) pages.
 *   - Element types: LAK_BF16 (bfloat16, float32 accumulation, outputs rounded to
 *     nearest even), LAK_F32, or LAK_FP8_E4M3 pools (rows in and out bfloat16).
 *   - Calls on one cache are not thread safe; calls that overlap on the device
 *     (different streams, same workspace) race.
 */
#ifndef LAK_H
#define LAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LAK_OK = 0,
  LAK_EINVAL = -1,       /* bad argument (null pointer, shape, range) */
  LAK_ENOPAGE = -2,      /* the page pool has no free page */
  LAK_EHIP = -3,         /* a HIP runtime call failed (includes earlier async faults) */
  LAK_EUNSUPPORTED = -4, /* valid but not built: head dim, group size, page size */
  LAK_ESTATE = -5        /* call out of order (e.g. no batch set by lak_seq_reset) */
} lak_status;

/* Pool element types.  LAK_FP8_E4M3: each (token, KV head) row of K and of V is
 * stored as D OCP E4M3 codes plus one float32 scale (scale = max|x| / 448, code =
 * round-to-nearest-even of x / scale; a row of zeros has scale 0).  The pages
 * name quantization as a technique to combine with DELTA ("Future Directions");
 * the format is the OCP 8-bit floating point E4M3 encoding.  Rows going in
 * (prefill, append, write_rows, k_new / v_new) and q / out are bfloat16 for such
 * a cache; attention runs on code * scale with float32 accumulation. */
typedef enum { LAK_BF16 = 0, LAK_F32 = 1, LAK_FP8_E4M3 = 2 } lak_dtype;

/* Head aggregation of per-token scores in a delta-layer.  MAX is the pages' rule
 * (a token's score is its largest weight over the heads); SUM adds the weights
 * instead. */
typedef enum { LAK_AGG_MAX = 0, LAK_AGG_SUM = 1 } lak_agg;

/* Which heads a delta-layer aggregates.  GROUP: the G query heads of each KV head,
 * one selection per (sequence, KV head).  ALL: all Hq query heads, one selection per
 * sequence shared by every KV head. */
typedef enum { LAK_SCOPE_GROUP = 0, LAK_SCOPE_ALL = 1 } lak_scope;

typedef struct lak_cache lak_cache; /* opaque; owns host metadata only */

/* Paged KV cache description.  Supported: head_dim 64 or 128; G = Hq / Hkv in
 * 1..16; page_size 16, 32 or 64.
 * Pools: one K and one V pool per layer, each num_pages pages of
 * [Hkv][P][D] elements (lak_pool_bytes() bytes); the in-page order of elements is
 * private to the library (written only by lak_kv_* calls).  page_table is
 * [max_batch][max_pages_per_seq] int32 physical page ids and seq_lens [max_batch]
 * int32 lengths, both device memory maintained by the library.
 * A descriptor whose page_table and seq_lens are both NULL (and pools NULL) gives
 * a metadata-only cache: the allocator runs on the host and nothing is sent to a
 * device (planning and tests without a GPU); attention calls on it fail. */
typedef struct {
  int32_t num_layers;
  int32_t max_batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages_per_seq;
  int32_t dtype;              /* lak_dtype */
  int64_t num_pages;          /* physical pages per pool */
  void* const* k_pools;       /* host array [num_layers] of device pointers */
  void* const* v_pools;       /* host array [num_layers] of device pointers */
  int32_t* page_table;        /* device [max_batch][max_pages_per_seq] */
  int32_t* seq_lens;          /* device [max_batch] */
} lak_cache_desc;

/* Bytes of one K (or V) pool: num_pages * Hkv * P * D * element size, plus
 * num_pages * Hkv * P * 4 for the scales of an fp8 pool; -1 if invalid. */
int64_t lak_pool_bytes(const lak_cache_desc* desc);

/* Validates `desc` and creates the host metadata.  No HIP call is made.
 * Errors: EINVAL (null, non-positive sizes, Hq not a multiple of Hkv),
 * EUNSUPPORTED (head dim, group size, page size outside the built set). */
lak_status lak_cache_create(const lak_cache_desc* desc, lak_cache** out);
lak_status lak_cache_destroy(lak_cache* cache);

/* Starts a new batch of `batch` sequences with prefilled lengths host_lens[b]
 * (>= 0).  Frees every page, then gives sequence b the pages for
 * host_lens[b] + reserve_tokens tokens (reserve_tokens >= 0 pre-reserves pages for
 * later decode steps so that lak_step_begin needs no new page).  Uploads the page
 * table rows and seq_lens on `stream` from host copies that the cache keeps until
 * the upload has completed (the next lak_seq_reset and lak_cache_destroy wait for
 * it; the call itself does not).  The caller then fills the cache with
 * lak_kv_prefill.  Errors: EINVAL, ENOPAGE (pool too small; the cache is then left
 * with no active batch). */
lak_status lak_seq_reset(lak_cache* cache, int32_t batch, const int32_t* host_lens,
                         int32_t reserve_tokens, void* stream);

/* Starts one decode step: T_b += 1 for every active sequence, taking a free page
 * for a sequence whose new token opens a page it has not reserved.  Enqueues one
 * small kernel (page-table entries passed by value) on `stream`.
 * Errors: ESTATE (no batch), EINVAL (a sequence would exceed max_pages_per_seq),
 * ENOPAGE (no free page; lengths unchanged). */
lak_status lak_step_begin(lak_cache* cache, void* stream);

/* Host mirror of the metadata.  lak_seq_lens_host copies B lengths into out
 * (cap >= B); lak_page_table_host copies the physical ids of sequence b's pages
 * (n_pages reserved pages, at most cap written). */
lak_status lak_seq_lens_host(const lak_cache* cache, int32_t* out, int32_t cap, int32_t* batch);
lak_status lak_page_table_host(const lak_cache* cache, int32_t b, int32_t* out, int32_t cap,
                               int32_t* n_pages);
int64_t lak_free_pages(const lak_cache* cache);

/* Workspace for the attention calls of this cache at its capacity (max_batch,
 * max_pages_per_seq): split-K partials, the delta-layer scratch (per head and
 * 16-token sub-tile, the maximum logit and fp16 weights relative to it, or the
 * (max, sum) pairs for SUM) and page-score scratch.  Device memory, any contents,
 * 256-byte aligned; calls read nothing a previous call left in it. */
size_t lak_workspace_bytes(const lak_cache* cache);

/* Writes this step's key and value of every active sequence into layer `layer` at
 * position T_b - 1 (call after lak_step_begin).  k_new, v_new: device
 * [B][Hkv][D] in the cache dtype.  DELTA keeps every token of the context in the
 * cache ("Methodology in Plain English": no token is evicted, so memory use is that
 * of full attention); this is how each decode step's token enters it. */
lak_status lak_kv_append(lak_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                         void* stream);

/* Writes prefilled keys/values: tokens [0, T_b) of every active sequence from
 * k, v: device [B][Hkv][t_stride][D] (token t of (b, kv head g) at
 * ((b * Hkv + g) * t_stride + t) * D).  t_stride >= max_b T_b. */
lak_status lak_kv_prefill(lak_cache* cache, int32_t layer, const void* k, const void* v,
                          int64_t t_stride, void* stream);

/* Overwrites n single (b, g, t) rows of layer `layer`: rows is device int32
 * [n][3] = (b, kv head, position < T_b), k_rows / v_rows device [n][D]
 * (v_rows may be NULL: keys only).  Rows out of range are skipped. */
lak_status lak_kv_write_rows(lak_cache* cache, int32_t layer, int32_t n, const int32_t* rows,
                             const void* k_rows, const void* v_rows, void* stream);

/* Reads tokens [t0, t0 + n) of (b, kv head g) of layer `layer` back in logical order
 * into k_out, v_out: device [n][D] (either may be NULL) in the pool's element type
 * (the E4M3 codes, one byte each, for an fp8 pool).  Requires t0 + n <= T_b. */
lak_status lak_kv_gather(lak_cache* cache, int32_t layer, int32_t b, int32_t g, int32_t t0,
                         int32_t n, void* k_out, void* v_out, void* stream);

/* fp8 pools only: the float32 scales of the same rows into k_out, v_out: device
 * [n] (either may be NULL).  Errors: EINVAL (not an fp8 cache, range). */
lak_status lak_kv_gather_scales(lak_cache* cache, int32_t layer, int32_t b, int32_t g, int32_t t0,
                                int32_t n, float* k_out, float* v_out, void* stream);

/* Full decode attention of layer `layer` (layers 0-1 and delta-layers attend to
 * the whole context): out[b][h] = sum_t p_t v_t over t < T_b with
 * p = softmax(sm_scale * <q[b][h], k_t>).  Split-K over pages plus a combine kernel.
 * k_new, v_new (both NULL, or both device [B][Hkv][D]): this step's key and value;
 * when given, the call also appends them at position T_b - 1, exactly as
 * lak_kv_append would before the call, inside its own decode kernel (one launch
 * fewer; fp8 caches encode the bfloat16 rows there).  The same holds for the
 * k_new / v_new arguments of lak_attn_delta_select and lak_attn_sparse.
 * lse may be NULL.  ws: lak_workspace_bytes() bytes of device memory. */
lak_status lak_attn_full(lak_cache* cache, int32_t layer, const void* q, const void* k_new,
                         const void* v_new, float sm_scale, void* out, float* lse, void* ws,
                         size_t ws_bytes, void* stream);

/* Delta-layer ("Methodology in Plain English" and "Main Findings", DELTA AI summary
 * page: a delta-layer attends to the whole context and renews the page choice of
 * the layers after it): the full attention of lak_attn_full (same out / lse), plus
 * the page selection it installs.  Per token t < T_b: a_t = AGG over the scope's heads of
 * exp(logit_{h,t} - lse_h); page score S_j = sum of a_t over the valid tokens of
 * page j.  Selection per row (row = (b, kv head) for GROUP, b for ALL): the last
 * `recency` pages, plus the `k_top` older pages of largest score (ties: lower page
 * index first), written as ascending logical page ids to
 * sel[row][0 .. count), -1 after; sel_count[row] = count = min(NP_b, k_top + recency).
 * sel: device int32 [B][R][sel_capacity], R = Hkv (GROUP) or 1 (ALL),
 * sel_capacity >= k_top + recency.  page_scores (nullable): device float32
 * [B][R][max_pages_per_seq], entries j >= NP_b left untouched; MAX scores come from
 * fp16 weights relative to each head's 16-token maximum (relative error <= 2^-11),
 * SUM scores are exact up to float32 rounding. */
lak_status lak_attn_delta_select(lak_cache* cache, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, float sm_scale, void* out, float* lse,
                                 int32_t k_top, int32_t recency,
                                 int32_t agg, int32_t scope, int32_t* sel, int32_t* sel_count,
                                 int32_t sel_capacity, float* page_scores, void* ws,
                                 size_t ws_bytes, void* stream);

/* The selection step alone on caller-supplied scores: page_scores device float32
 * [B][R][max_pages_per_seq] (row NP_b from seq_lens); same rule and outputs as
 * lak_attn_delta_select.  Scores are compared as float32; negative and NaN scores
 * count as 0. */
lak_status lak_page_select(lak_cache* cache, const float* page_scores, int32_t scope,
                           int32_t k_top, int32_t recency, int32_t* sel, int32_t* sel_count,
                           int32_t sel_capacity, void* stream);

/* Sparse layer ("Methodology in Plain English", DELTA AI summary page: the layers
 * after a delta-layer attend only to the tokens of the pages it chose): attention of
 * every query head over the tokens t < T_b of the pages listed in the selection of
 * its KV head (sel / sel_count as written by
 * lak_attn_delta_select with the same scope; entries outside [0, NP_b) are
 * skipped; duplicates are the caller's error).  The softmax is over those tokens
 * only.  A row with no valid page yields out = 0 and lse = -inf. */
lak_status lak_attn_sparse(lak_cache* cache, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, float sm_scale, const int32_t* sel,
                           const int32_t* sel_count, int32_t sel_capacity, int32_t scope, void* out,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): lak_attn_sparse with the
 * same arguments, outputs and errors, minus the workspace.  Its split partials go to
 * a static device buffer of 16 MiB that the library owns (one copy per GPU, kept
 * until the process ends; its address is looked up once per device, on the first
 * call with that device current).  The call itself allocates nothing and only
 * launches kernels.  It needs align256(B * Hq * S * D * 4) + B * Hq * S * 8 bytes of
 * it, S = the call's splits per row (the library aims at about 1024 workgroups in
 * all, S ~ 1024 / (B * Hkv), with at most 256 selection entries per split); a call
 * that would need more than 16 MiB fails with LAK_EINVAL before anything is
 * enqueued.  Every call on one GPU shares that buffer, and its
 * kernels read only what the same call wrote: calls that may overlap on the device
 * (different streams or threads) race and must be serialised by the caller. */
lak_status lak_attn_sparse_noalloc(lak_cache* cache, int32_t layer, const void* q, const void* k_new,
                                   const void* v_new, float sm_scale, const int32_t* sel,
                                   const int32_t* sel_count, int32_t sel_capacity, int32_t scope, void* out,
                                   float* lse, void* stream);

/* One decode step of a whole attention stack (the three-tier schedule of
 * "Methodology in Plain English": full layers, delta-layers that renew the page
 * choice, sparse layers over the most recent choice, renewed at every token).
 * Performs lak_step_begin, then for every layer l in order: the attention call of
 * its tier (full / delta-select / sparse with the selection of the latest
 * delta-layer before l), appending k_new[l] / v_new[l] inside the call.  All host
 * arrays have num_layers entries of device pointers; lse[l] may be NULL; sel[l] /
 * sel_count[l] are used (and required) for delta layers only, shaped as in
 * lak_attn_delta_select with sel_capacity >= k_top + recency.  Every argument is
 * validated before anything is enqueued or any length changes; errors: EINVAL (bad
 * tier, a sparse layer before any delta-layer, NULL pointer), plus those of
 * lak_step_begin.  Past validation only a failing kernel launch (LAK_EHIP) can end
 * the call early: the step has then begun (lengths advanced, page-table update
 * enqueued) and the layers before the failing one are enqueued; such a failure
 * means the device is unusable, not that the step can be retried. */
typedef struct {
  int32_t num_layers;
  const int32_t* tiers;        /* host [num_layers]: 0 full, 1 delta, 2 sparse */
  const void* const* q;        /* host [num_layers] of device [B][Hq][D] */
  const void* const* k_new;    /* host [num_layers] of device [B][Hkv][D] */
  const void* const* v_new;    /* host [num_layers] of device [B][Hkv][D] */
  void* const* out;            /* host [num_layers] of device [B][Hq][D] */
  float* const* lse;           /* host [num_layers] of device [B][Hq] (entries may be NULL) */
  int32_t* const* sel;         /* host [num_layers]: delta layers' device selection buffers */
  int32_t* const* sel_count;   /* host [num_layers]: delta layers' device counts */
  int32_t sel_capacity;
  float sm_scale;
  int32_t k_top, recency, agg, scope;
  void* const* trace_before;   /* NULL, or host [num_layers] of hipEvent_t (entries may be NULL): */
  void* const* trace_after;    /* recorded around layer l's decode kernel as lak_trace_decode does */
} lak_stack_step_desc;

lak_status lak_stack_step(lak_cache* cache, const lak_stack_step_desc* step, void* ws, size_t ws_bytes,
                          void* stream);

/* Tracing: while set, every attention call on `cache` attaches `before` and `after`
 * (hipEvent_t created by the caller, with timing) to the dispatch of its split-K
 * decode kernel on its stream (hipExtLaunchKernelGGL), so that they take the
 * kernel's start and end times and hipEventElapsedTime gives its execution time.
 * Events created with hipEventDisableSystemFence (read only after a device
 * synchronisation) add the least to the stream's time.
 * NULL, NULL stops it.  Errors: EINVAL if exactly one event is NULL. */
lak_status lak_trace_decode(lak_cache* cache, void* before, void* after);

/* Reason for the last failing call of this thread ("" if none). */
const char* lak_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LAK_H */
