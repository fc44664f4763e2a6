// C ABI of the layer-aware KV decode-attention library: argument validation, the
// host page allocator, workspace layout, split planning and kernel launches.
// See include/lak.h for the contract of every entry point.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "lak.h"
#include "lak_internal.h"

using namespace lak;

namespace {

thread_local std::string g_err;

lak_status fail(lak_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// Success leaves the last error message in place (it describes the last failure).
lak_status ok() { return LAK_OK; }

lak_status hip_fail(hipError_t e, const char* where) {
  return fail(LAK_EHIP, "%s: %s", where, hipGetErrorString(e));
}

// Workgroups a split-K launch aims for and the fewest 16-token sub-tiles one workgroup
// is given.  Full tier: three per CU of a 256-CU part, one round (at batch 16, 64k
// context the all-full stack ran 1.8% faster than at 1024 and 1-6% slower at 512, 640
// and 896, alternated in one process; batch 8, 16k context 2.6% faster than 1024).
// Sparse tier: four per CU (768 and 1536 were 0.4% and 2.2% slower at batch 16).
constexpr int kTargetWgsFull = 768;
constexpr int kTargetWgsSparse = 1024;
// Delta tier.  Where a split's LDS stage of page-score scratch limits a CU to fewer
// than four workgroups (MAX aggregation at long contexts), the launch aims at the fewest
// workgroups whose stage still leaves room for three; otherwise at 1.5 rounds of four
// per CU (kTargetWgsDeltaLong) when that still gives a workgroup kDeltaLongMinSubtiles
// sub-tiles, else at one round (kTargetWgsDeltaMin).  Alternated in one process: batch
// 16, 64k context, G 7, MAX: 1280 workgroups (splits of up to 209 pages, a 53.5 KiB
// stage) ran the stack 0.8-0.9% faster than 1536 and 0.6-4% faster than 1152-1408;
// SUM (a small stage): 1536 0.6-2.7% faster than 1024-2048; batch 8, 16k context:
// 1024 1.6% (MAX) and 2.9% (SUM) faster than 1536.
constexpr int kTargetWgsDeltaMin = 1024;
constexpr int kTargetWgsDeltaLong = 1536;
constexpr int kDeltaLongMinSubtiles = 64;
constexpr int kDeltaWgsPerCu = 3;
// Ragged batches (the longest row more than 1.1x the mean) on the full and delta tiers:
// splits of a uniform batch end together in one workgroup round, those of unequal rows
// do not, and smaller splits then keep the CUs busy to the end (workload of 32 rows of
// 256-1024 pages: full 448 -> 410 us, delta 486 -> 467 us).
constexpr int kTargetWgsRagged = 3072;
constexpr int kMinSubtilesPerWg = 8;
// Each of the 4 waves of a decode workgroup keeps the page ids of its items in one
// register per lane (two for the full tier), so a split holds at most 4 * 64 items
// (4 * 128).  The full tier's wider cap keeps a one-page-longer context at one
// workgroup round (4097 pages: 16 splits of 257 instead of 17 of 256).
constexpr int kMaxItemsPerSplit = 256;
constexpr int kMaxItemsPerSplitFull = 512;
// MAX page scoring: a block takes 1024-4096 consecutive tokens of a score row, as many as
// keep the launch near kScoreTargetWgs blocks.  Alternated in one process: batch 8, 16k
// context (512 blocks at 1024 tokens) ran the stack 2.0% faster than at 4096 (128
// blocks); batch 16, 64k context stays at 4096 (1024 blocks; 18.7 -> 17.9 us per delta
// layer against 2048 across processes, equal in one); batch 32 ragged to 32k stays at
// 4096 (1024 tokens: 1.6% slower).
constexpr int kScoreTokensMin = 1024;
constexpr int kScoreTokensMax = 4096;
constexpr int kScoreTargetWgs = 1024;

int esize(int dtype) { return dtype == LAK_BF16 ? 2 : (dtype == LAK_FP8_E4M3 ? 1 : 4); }

bool valid_dtype(int dtype) { return dtype == LAK_BF16 || dtype == LAK_F32 || dtype == LAK_FP8_E4M3; }

// Bytes of one pool's element codes; fp8 pools hold one float32 scale per token row after them.
int64_t code_bytes(const lak_cache_desc& d) {
  return d.num_pages * d.num_kv_heads * (int64_t)d.page_size * d.head_dim * esize(d.dtype);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  const int x = std::atoi(v);
  return (x < lo || x > hi) ? dflt : x;
}

}  // namespace

int lak::tune_decode_batch(int mode) {
  // 0: chosen per launch (launch_decode_t)
  static const int full = env_int("LAK_TUNE_DECODE_BATCH", 1, 1, 2);
  static const int delta = env_int("LAK_TUNE_DELTA_BATCH", 0, 0, 2);
  static const int sparse = env_int("LAK_TUNE_SPARSE_BATCH", 0, 0, 4);
  return mode == MODE_SPARSE ? (sparse == 3 ? 2 : sparse) : (mode == MODE_DELTA ? delta : full);
}

int lak::tune_target_wgs(int mode, int64_t work, size_t stage_per_item, int subtiles_per_item) {
  static const int full = env_int("LAK_TUNE_TARGET_WGS", kTargetWgsFull, 64, 65536);
  static const int sparse = env_int("LAK_TUNE_SPARSE_WGS", kTargetWgsSparse, 64, 65536);
  static const int delta = env_int("LAK_TUNE_DELTA_WGS", 0, 64, 65536);  // 0: by the stage size
  if (mode != MODE_DELTA) return mode == MODE_SPARSE ? sparse : full;
  if (delta) return delta;
  // stage bytes that leave room for three, less 1 KiB per workgroup for the allocation granularity
  const size_t per_wg = kLdsBytesPerCu / kDeltaWgsPerCu - 1024;
  const int64_t items = std::max<int64_t>(1, (int64_t)(per_wg / std::max<size_t>(stage_per_item, 1)));
  const int64_t lds_wgs = (work + items - 1) / items;
  if (lds_wgs > kTargetWgsDeltaMin) return (int)std::min<int64_t>(lds_wgs, 65536);
  const int64_t subtiles = work * std::max(subtiles_per_item, 1);
  return subtiles >= (int64_t)kTargetWgsDeltaLong * kDeltaLongMinSubtiles ? kTargetWgsDeltaLong : kTargetWgsDeltaMin;
}

int lak::tune_ragged_wgs() {
  static const int v = env_int("LAK_TUNE_RAGGED_WGS", kTargetWgsRagged, 64, 65536);
  return v;
}

int lak::tune_min_subtiles() {
  static const int v = env_int("LAK_TUNE_MIN_SUBTILES", kMinSubtilesPerWg, 1, 256);
  return v;
}

int lak::tune_score_tokens(int64_t row_tokens) {
  // whole rounds of 256 threads x 4 tokens, so that no page straddles two blocks (P <= 64)
  static const int v = env_int("LAK_TUNE_SCORE_TOKENS", 0, 1024, 65536);  // 0: by the call's size
  if (v) return v - v % 1024;
  const int64_t per = (row_tokens + kScoreTargetWgs - 1) / kScoreTargetWgs;
  const int64_t t = (per + 1023) / 1024 * 1024;
  return (int)std::min<int64_t>(kScoreTokensMax, std::max<int64_t>(kScoreTokensMin, t));
}

int lak::tune_topk_wave_kpl() {
  // 0 by default: the workgroup selector measured faster at every row length tried
  // (512 to 8000 pages, 16 x 4 rows: 7.6-17 us against 9.0-42.6 us for one wave per row)
  static const int v = env_int("LAK_TUNE_TOPK_WAVE_KPL", 0, 0, 128);
  return v;
}

int lak::tune_delta_lds() {
  static const int v = env_int("LAK_TUNE_DELTA_LDS", 1, 0, 1);
  return v;
}

// Static device scratch of lak_attn_sparse_noalloc: the split partials of one call, in
// memory the library itself owns (one copy per GPU, held until the process ends), for
// callers that cannot allocate.  Host code never uses this name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress (noalloc_scratch).
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

struct lak_cache {
  lak_cache_desc d;
  std::vector<void*> kp, vp;
  bool host_only = false;
  int batch = -1;
  std::vector<int32_t> lens;
  std::vector<std::vector<int32_t>> pages;
  std::vector<int32_t> free_list;  // stack; back() is handed out next
  // host sources of lak_seq_reset's uploads: kept until `staging_done` (recorded after
  // the copies) has completed, so that the call need not wait for them
  std::vector<int32_t> table_staging;
  std::vector<int32_t> lens_staging;
  hipEvent_t staging_done = nullptr;
  int s_cap = 0;
  hipEvent_t trace_before = nullptr, trace_after = nullptr;

  int max_np() const {
    int m = 0;
    for (int b = 0; b < batch; ++b) m = std::max(m, (lens[b] + d.page_size - 1) / d.page_size);
    return m;
  }
  int max_len() const {
    int m = 0;
    for (int b = 0; b < batch; ++b) m = std::max(m, lens[b]);
    return m;
  }
  void reset_free_list() {
    free_list.clear();
    free_list.reserve((size_t)d.num_pages);
    for (int64_t p = d.num_pages - 1; p >= 0; --p) free_list.push_back((int32_t)p);
    for (auto& v : pages) v.clear();
  }
};

namespace {

struct WsLayout {
  size_t o_part, ml_part, delta, scores, total;
};

WsLayout ws_layout(const lak_cache* c) {
  const auto& d = c->d;
  WsLayout w;
  size_t off = 0;
  // split partials are [B][Hq][S] with S the call's split count: B * S <= s_cap
  const size_t part = (size_t)d.num_q_heads * c->s_cap;
  w.o_part = off;
  off = align256(off + part * d.head_dim * sizeof(float));
  w.ml_part = off;
  off = align256(off + part * 2 * sizeof(float));
  // delta scratch, per (b, g, 16-token sub-tile) of the cache's capacity: the MAX block
  // (G x 16 fp16 relative weights, then G float maxima, max_block_bytes(G) bytes) or the
  // SUM (max, sum) float pairs of Gp heads (Gp = G rounded up to even)
  w.delta = off;
  const int G = d.num_q_heads / d.num_kv_heads;
  const size_t gp = (size_t)(G + (G & 1));
  const size_t subs = (size_t)d.max_batch * d.num_kv_heads * ((size_t)d.max_pages_per_seq * d.page_size / 16);
  off = align256(off + subs * std::max((size_t)max_block_bytes(G), gp * 2 * sizeof(float)));
  w.scores = off;
  off = align256(off + (size_t)d.max_batch * d.num_kv_heads * d.max_pages_per_seq * sizeof(float));
  w.total = off;
  return w;
}

// Items (pages or selection entries) per split.  `work` is the total over the call's
// rows (per-row item counts summed: a ragged batch gives its long rows more splits),
// `max_items` the longest row's count and `max_splits` the most splits a row may use
// (the partial buffers hold max_splits per row).
int plan_pps(int64_t work, int max_items, int max_splits, int subtiles_per_page, int mode, bool ragged,
             size_t stage_per_item) {
  const int base = tune_target_wgs(mode, work, stage_per_item, subtiles_per_page);
  const int target = (ragged && mode != MODE_SPARSE) ? std::max(tune_ragged_wgs(), base) : base;
  int pps = (int)((work + target - 1) / target);
  pps = std::max(pps, (max_items + max_splits - 1) / std::max(max_splits, 1));
  const int min_sub = tune_min_subtiles();
  const int min_pps = (min_sub + subtiles_per_page - 1) / subtiles_per_page;
  return std::min(std::max(std::max(pps, min_pps), 1), mode == MODE_FULL ? kMaxItemsPerSplitFull : kMaxItemsPerSplit);
}

// Device address of the current GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

lak_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LAK_EUNSUPPORTED, "device ordinal %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LAK_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LAK_OK;
}

#ifdef LAK_DEBUG_CHECKS
// Debug builds: after every allocation, every page id held by an active sequence is a
// valid physical page (< num_pages), no page is held twice or also free, and held plus
// free pages make up the pool.  A violation is a library bug: report and abort.
void debug_check_pages(const lak_cache* c) {
  const int64_t n = c->d.num_pages;
  std::vector<uint8_t> seen((size_t)n, 0);
  int64_t held = 0;
  auto bad = [&](const char* what, long long v) {
    std::fprintf(stderr, "lak debug check: %s (%lld)\n", what, v);
    std::abort();
  };
  for (int b = 0; b < std::max(c->batch, 0); ++b) {
    if ((int64_t)c->pages[b].size() * c->d.page_size < c->lens[b]) bad("sequence shorter in pages than its length", b);
    for (int32_t p : c->pages[b]) {
      if (p < 0 || p >= n) bad("page id outside the pool", p);
      if (seen[(size_t)p]++) bad("page held twice", p);
      ++held;
    }
  }
  for (int32_t p : c->free_list) {
    if (p < 0 || p >= n) bad("free page id outside the pool", p);
    if (seen[(size_t)p]++) bad("page both free and held", p);
  }
  if (held + (int64_t)c->free_list.size() != n) bad("pages lost", n - held - (int64_t)c->free_list.size());
}
#define LAK_DEBUG_CHECK_PAGES(c) debug_check_pages(c)
#else
#define LAK_DEBUG_CHECK_PAGES(c) ((void)0)
#endif

lak_status check_cache(const lak_cache* c, bool need_device) {
  if (!c) return fail(LAK_EINVAL, "cache is NULL");
  if (c->batch < 0) return fail(LAK_ESTATE, "no active batch: call lak_seq_reset first");
  if (need_device && c->host_only) return fail(LAK_ESTATE, "metadata-only cache has no device buffers");
  return LAK_OK;
}

lak_status check_layer(const lak_cache* c, int layer) {
  if (layer < 0 || layer >= c->d.num_layers)
    return fail(LAK_EINVAL, "layer %d out of range [0, %d)", layer, c->d.num_layers);
  if (!c->kp[layer] || !c->vp[layer]) return fail(LAK_EINVAL, "pool of layer %d is NULL", layer);
  return LAK_OK;
}

KvGeom geom(const lak_cache* c) {
  KvGeom g;
  g.hkv = c->d.num_kv_heads;
  g.d = c->d.head_dim;
  g.page = c->d.page_size;
  g.max_pages = c->d.max_pages_per_seq;
  g.esz = esize(c->d.dtype);
  g.scale_off = code_bytes(c->d);
  return g;
}

lak_status check_ws(const lak_cache* c, const void* ws, size_t ws_bytes) {
  const size_t need = ws_layout(c).total;
  if (!ws) return fail(LAK_EINVAL, "workspace is NULL");
  if (ws_bytes < need) return fail(LAK_EINVAL, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  if (((uintptr_t)ws & 255) != 0) return fail(LAK_EINVAL, "workspace not 256-byte aligned");
  return LAK_OK;
}

// Bytes of the split partials (o, then (max, sum)) of a call with `splits` splits per row.
size_t partial_bytes(const lak_cache* c, int splits) {
  const size_t rows = (size_t)c->batch * c->d.num_q_heads * splits;
  return align256(rows * c->d.head_dim * sizeof(float)) + rows * 2 * sizeof(float);
}

// Runs the split-K decode plus combine of one tier.
// With `defer_combine` the combine arguments are returned there instead of launched
// (the delta layer combines inside its page-scoring launch).  With `parts` the split
// partials go there (at most `parts_cap` bytes, checked before anything is launched)
// instead of the workspace, which is then not used.
lak_status run_attention(lak_cache* c, int layer, int mode, const void* q, const void* k_new,
                         const void* v_new, float sm_scale, void* out, float* lse, const int32_t* sel,
                         const int32_t* sel_count, int sel_cap, int sel_rows, void* ws, hipStream_t st,
                         int agg = LAK_AGG_MAX, CombineArgs* defer_combine = nullptr, void* parts = nullptr,
                         size_t parts_cap = 0) {
  const auto& d = c->d;
  const WsLayout w = ws_layout(c);
  char* wsb = static_cast<char*>(ws);
  const int spp = d.page_size / 16;
  // items per row: the row's pages (a sparse row: at most sel_cap selection entries)
  int max_items = 0;
  int64_t work = 0;
  for (int b = 0; b < c->batch; ++b) {
    int items = (c->lens[b] + d.page_size - 1) / d.page_size;
    if (mode == MODE_SPARSE) items = std::min(items, sel_cap);
    max_items = std::max(max_items, items);
    work += (int64_t)items * d.num_kv_heads;
  }
  // ragged: the longest row holds more than 1.1x the mean row's items
  const bool ragged = (int64_t)max_items * c->batch * d.num_kv_heads * 10 > work * 11;
  const int G = d.num_q_heads / d.num_kv_heads;
  const size_t stage_per_item = delta_stage_bytes(1, d.page_size, G, agg == LAK_AGG_SUM);
  const int pps = plan_pps(work, max_items, c->s_cap / std::max(c->batch, 1), spp, mode, ragged, stage_per_item);
  const int splits = (max_items + pps - 1) / pps;
  if ((int64_t)splits * c->batch > c->s_cap)
    return fail(LAK_EINVAL, "internal: %d splits x %d rows exceed capacity %d", splits, c->batch, c->s_cap);
  if (parts && partial_bytes(c, splits) > parts_cap)
    return fail(LAK_EINVAL,
                "split partials need %zu bytes, more than the %zu-byte static scratch (batch %d, %d splits)",
                partial_bytes(c, splits), parts_cap, c->batch, splits);

  DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  hipError_t e = hipSuccess;
  if (d.dtype == LAK_FP8_E4M3) {
    a.k_scale = reinterpret_cast<const float*>(static_cast<const char*>(c->kp[layer]) + code_bytes(d));
    a.v_scale = reinterpret_cast<const float*>(static_cast<const char*>(c->vp[layer]) + code_bytes(d));
  }
  a.k_pool = c->kp[layer];
  a.v_pool = c->vp[layer];
  a.page_table = d.page_table;
  a.seq_lens = d.seq_lens;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.sm_scale = sm_scale;
  a.hq = d.num_q_heads;
  a.hkv = d.num_kv_heads;
  a.page = d.page_size;
  a.max_pages = d.max_pages_per_seq;
  a.pps = pps;
  a.s_cap = splits;
  a.sel = sel;
  a.sel_count = sel_count;
  a.sel_cap = sel_cap;
  a.sel_rows = sel_rows;
  if (parts) {
    char* pb = static_cast<char*>(parts);
    a.o_part = reinterpret_cast<float*>(pb);
    a.ml_part = reinterpret_cast<float*>(pb + align256((size_t)c->batch * d.num_q_heads * splits * d.head_dim *
                                                       sizeof(float)));
  } else {
    a.o_part = reinterpret_cast<float*>(wsb + w.o_part);
    a.ml_part = reinterpret_cast<float*>(wsb + w.ml_part);
  }
  if (mode == MODE_DELTA) {
    a.pairs = reinterpret_cast<float*>(wsb + w.delta);
    a.rel_blk = reinterpret_cast<uint8_t*>(wsb + w.delta);
  }
  a.lds_stage = (mode == MODE_DELTA && tune_delta_lds() && pps * stage_per_item <= 64 * 1024) ? 1 : 0;
  a.sum_pairs = (mode == MODE_DELTA && agg == LAK_AGG_SUM) ? 1 : 0;
  a.t_pad = (int64_t)d.max_pages_per_seq * d.page_size;
  e = launch_decode(d.dtype, mode, d.head_dim, a, splits, c->batch, st, c->trace_before, c->trace_after);
  if (e != hipSuccess) return hip_fail(e, "decode launch");

  CombineArgs cb;
  std::memset(&cb, 0, sizeof(cb));
  cb.o_part = a.o_part;
  cb.ml_part = a.ml_part;
  cb.seq_lens = d.seq_lens;
  cb.sel_count = (mode == MODE_SPARSE) ? sel_count : nullptr;
  cb.sel_cap = sel_cap;
  cb.sel_rows = sel_rows;
  cb.hq = d.num_q_heads;
  cb.hkv = d.num_kv_heads;
  cb.page = d.page_size;
  cb.pps = pps;
  cb.s_cap = splits;
  cb.splits = splits;
  cb.out = out;
  cb.lse = lse;
  if (defer_combine) {
    *defer_combine = cb;
    return ok();
  }
  e = launch_combine(d.dtype, d.head_dim, cb, c->batch, st);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return ok();
}

lak_status run_select(lak_cache* c, const float* scores, int scope, int k_top, int recency,
                      int32_t* sel, int32_t* sel_count, int sel_cap, hipStream_t st) {
  TopkArgs t;
  t.scores = scores;
  t.seq_lens = c->d.seq_lens;
  t.sel = sel;
  t.sel_count = sel_count;
  t.rows_per_seq = scope == LAK_SCOPE_GROUP ? c->d.num_kv_heads : 1;
  t.page = c->d.page_size;
  t.max_pages = c->d.max_pages_per_seq;
  t.k_top = k_top;
  t.recency = recency;
  t.sel_cap = sel_cap;
  t.max_np = c->max_np();
  hipError_t e = launch_topk(t, c->batch, st);
  if (e != hipSuccess) return hip_fail(e, "top-k launch");
  return ok();
}

lak_status check_select_args(const lak_cache* c, int scope, int k_top, int recency, const int32_t* sel,
                             const int32_t* sel_count, int sel_cap) {
  if (scope != LAK_SCOPE_GROUP && scope != LAK_SCOPE_ALL) return fail(LAK_EINVAL, "bad scope %d", scope);
  if (k_top < 0 || recency < 0) return fail(LAK_EINVAL, "k_top and recency must be >= 0");
  if ((int64_t)k_top + recency > sel_cap)
    return fail(LAK_EINVAL, "sel_capacity %d < k_top + recency = %lld", sel_cap, (long long)k_top + recency);
  if (!sel || !sel_count) return fail(LAK_EINVAL, "sel / sel_count is NULL");
  (void)c;
  return LAK_OK;
}

}  // namespace

extern "C" {

int64_t lak_pool_bytes(const lak_cache_desc* d) {
  if (!d || d->num_pages <= 0 || d->num_kv_heads <= 0 || d->page_size <= 0 || d->head_dim <= 0 ||
      !valid_dtype(d->dtype))
    return -1;
  const int64_t scales = d->dtype == LAK_FP8_E4M3 ? d->num_pages * d->num_kv_heads * (int64_t)d->page_size * 4 : 0;
  return code_bytes(*d) + scales;
}

lak_status lak_cache_create(const lak_cache_desc* desc, lak_cache** out) {
  if (!desc || !out) return fail(LAK_EINVAL, "desc/out is NULL");
  const lak_cache_desc& d = *desc;
  if (d.num_layers <= 0 || d.max_batch <= 0 || d.num_q_heads <= 0 || d.num_kv_heads <= 0 ||
      d.head_dim <= 0 || d.page_size <= 0 || d.max_pages_per_seq <= 0 || d.num_pages <= 0)
    return fail(LAK_EINVAL, "all sizes must be positive");
  if (d.num_q_heads % d.num_kv_heads != 0)
    return fail(LAK_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", d.num_q_heads, d.num_kv_heads);
  if (!valid_dtype(d.dtype)) return fail(LAK_EINVAL, "bad dtype %d", d.dtype);
  if (d.num_pages > 0x7FFFFFFF) return fail(LAK_EINVAL, "num_pages exceeds int32 page ids");
  const int G = d.num_q_heads / d.num_kv_heads;
  if (G > 16) return fail(LAK_EUNSUPPORTED, "group size %d > 16", G);
  if (d.head_dim != 64 && d.head_dim != 128) return fail(LAK_EUNSUPPORTED, "head_dim %d (built: 64, 128)", d.head_dim);
  if (d.page_size != 16 && d.page_size != 32 && d.page_size != 64)
    return fail(LAK_EUNSUPPORTED, "page_size %d (built: 16, 32, 64)", d.page_size);
  if ((int64_t)d.max_pages_per_seq * d.page_size > 0x7FFFFFFF)
    return fail(LAK_EINVAL, "max_pages_per_seq * page_size exceeds int32 positions");
  const bool host_only = !d.page_table && !d.seq_lens;
  if (!host_only) {
    if (!d.page_table || !d.seq_lens) return fail(LAK_EINVAL, "page_table and seq_lens must both be set");
    if (!d.k_pools || !d.v_pools) return fail(LAK_EINVAL, "k_pools / v_pools arrays are NULL");
  }
  lak_cache* c = new lak_cache();
  c->d = d;
  c->host_only = host_only;
  c->kp.assign(d.num_layers, nullptr);
  c->vp.assign(d.num_layers, nullptr);
  if (!host_only)
    for (int l = 0; l < d.num_layers; ++l) {
      c->kp[l] = d.k_pools[l];
      c->vp[l] = d.v_pools[l];
    }
  c->d.k_pools = nullptr;
  c->d.v_pools = nullptr;
  c->pages.resize(d.max_batch);
  c->lens.assign(d.max_batch, 0);
  c->reset_free_list();
  // Bound on B * S over all calls: with pps >= ceil(R * M / target) (R = B * Hkv rows of
  // at most M items) S <= target / R + 1, and with pps capped at kMaxItemsPerSplit
  // S <= M / kMaxItemsPerSplit + 1.
  {
    // (the delta tier's target grows with the call's work; where it passes this bound the
    // split count is capped by the partial buffers and the splits grow instead)
    const int tiers = std::max(tune_target_wgs(MODE_FULL, 0, 0, 1), tune_target_wgs(MODE_SPARSE, 0, 0, 1));
    const int tmax = std::max(std::max(tiers, std::max(kTargetWgsDeltaLong, 2048)), tune_ragged_wgs());
    c->s_cap = (tmax + d.num_kv_heads - 1) / d.num_kv_heads +
               d.max_batch * ((d.max_pages_per_seq + kMaxItemsPerSplit - 1) / kMaxItemsPerSplit + 2);
  }
  *out = c;
  return ok();
}

lak_status lak_cache_destroy(lak_cache* c) {
  if (c && c->staging_done) {
    // the last upload may still read the staging vectors freed with the cache
    (void)hipEventSynchronize(c->staging_done);
    (void)hipEventDestroy(c->staging_done);
  }
  delete c;
  return ok();
}

lak_status lak_seq_reset(lak_cache* c, int32_t batch, const int32_t* host_lens, int32_t reserve_tokens,
                         void* stream) {
  if (!c) return fail(LAK_EINVAL, "cache is NULL");
  if (batch < 0 || batch > c->d.max_batch) return fail(LAK_EINVAL, "batch %d outside [0, %d]", batch, c->d.max_batch);
  if (batch > 0 && !host_lens) return fail(LAK_EINVAL, "host_lens is NULL");
  if (reserve_tokens < 0) return fail(LAK_EINVAL, "reserve_tokens < 0");
  const int P = c->d.page_size;
  int64_t need = 0;
  for (int b = 0; b < batch; ++b) {
    if (host_lens[b] < 0) return fail(LAK_EINVAL, "host_lens[%d] < 0", b);
    const int64_t np = ((int64_t)host_lens[b] + reserve_tokens + P - 1) / P;
    if (np > c->d.max_pages_per_seq)
      return fail(LAK_EINVAL, "sequence %d needs %lld pages > max_pages_per_seq %d", b, (long long)np,
                  c->d.max_pages_per_seq);
    need += np;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (c->staging_done) {
    // the previous call's uploads read the staging vectors refilled below (complete
    // long before in any real use: this returns at once)
    hipError_t e = hipEventSynchronize(c->staging_done);
    if (e != hipSuccess) return hip_fail(e, "previous page table upload");
  }
  c->batch = -1;
  c->reset_free_list();
  if (need > (int64_t)c->free_list.size())
    return fail(LAK_ENOPAGE, "batch needs %lld pages, pool has %lld", (long long)need, (long long)c->d.num_pages);
  for (int b = 0; b < batch; ++b) {
    const int np = (int)(((int64_t)host_lens[b] + reserve_tokens + P - 1) / P);
    c->pages[b].resize(np);
    for (int i = 0; i < np; ++i) {
      c->pages[b][i] = c->free_list.back();
      c->free_list.pop_back();
    }
    c->lens[b] = host_lens[b];
  }
  c->batch = batch;
  LAK_DEBUG_CHECK_PAGES(c);
  if (c->host_only || batch == 0) return ok();
  const int mp = c->d.max_pages_per_seq;
  c->table_staging.assign((size_t)batch * mp, 0);
  for (int b = 0; b < batch; ++b)
    std::copy(c->pages[b].begin(), c->pages[b].end(), c->table_staging.begin() + (size_t)b * mp);
  c->lens_staging.assign(c->lens.begin(), c->lens.begin() + batch);
  hipError_t e = hipSuccess;
  if (!c->staging_done) e = hipEventCreateWithFlags(&c->staging_done, hipEventDisableTiming);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->d.page_table, c->table_staging.data(), c->table_staging.size() * 4,
                       hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->d.seq_lens, c->lens_staging.data(), c->lens_staging.size() * 4,
                       hipMemcpyHostToDevice, st);
  // the staging vectors outlive the copies: the next reset and destroy wait for this
  if (e == hipSuccess) e = hipEventRecord(c->staging_done, st);
  if (e != hipSuccess) return hip_fail(e, "page table upload");
  return ok();
}

lak_status lak_step_begin(lak_cache* c, void* stream) {
  lak_status s = check_cache(c, false);
  if (s != LAK_OK) return s;
  const int P = c->d.page_size;
  // plan first: nothing changes unless every sequence gets its page
  std::vector<int> needs;
  for (int b = 0; b < c->batch; ++b) {
    const int t = c->lens[b] + 1;
    const int np = (t + P - 1) / P;
    if (np > c->d.max_pages_per_seq)
      return fail(LAK_EINVAL, "sequence %d would exceed max_pages_per_seq %d", b, c->d.max_pages_per_seq);
    if (np > (int)c->pages[b].size()) needs.push_back(b);
  }
  if (needs.size() > c->free_list.size())
    return fail(LAK_ENOPAGE, "step needs %zu new pages, %zu free", needs.size(), c->free_list.size());
  std::vector<int32_t> nb, nlp, npg;
  for (int b : needs) {
    const int32_t p = c->free_list.back();
    c->free_list.pop_back();
    nb.push_back(b);
    nlp.push_back((int32_t)c->pages[b].size());
    npg.push_back(p);
    c->pages[b].push_back(p);
  }
  for (int b = 0; b < c->batch; ++b) c->lens[b] += 1;
  LAK_DEBUG_CHECK_PAGES(c);
  if (c->host_only) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  size_t i = 0;
  do {
    StepUpdate u;
    std::memset(&u, 0, sizeof(u));
    u.n = (int32_t)std::min<size_t>(kStepMax, nb.size() - i);
    for (int k = 0; k < u.n; ++k) {
      u.b[k] = nb[i + k];
      u.lp[k] = nlp[i + k];
      u.page[k] = npg[i + k];
    }
    i += u.n;
    u.batch = (i >= nb.size()) ? c->batch : 0;
    hipError_t e = launch_step_update(u, c->d.page_table, c->d.seq_lens, c->d.max_pages_per_seq, st);
    if (e != hipSuccess) return hip_fail(e, "step update launch");
  } while (i < nb.size());
  return ok();
}

lak_status lak_seq_lens_host(const lak_cache* c, int32_t* out, int32_t cap, int32_t* batch) {
  if (!c || !out) return fail(LAK_EINVAL, "NULL argument");
  const int B = std::max(c->batch, 0);
  if (cap < B) return fail(LAK_EINVAL, "cap %d < batch %d", cap, B);
  for (int b = 0; b < B; ++b) out[b] = c->lens[b];
  if (batch) *batch = c->batch;
  return ok();
}

lak_status lak_page_table_host(const lak_cache* c, int32_t b, int32_t* out, int32_t cap, int32_t* n_pages) {
  if (!c || !out || !n_pages) return fail(LAK_EINVAL, "NULL argument");
  if (b < 0 || b >= c->batch) return fail(LAK_EINVAL, "sequence %d not active", b);
  const auto& v = c->pages[b];
  *n_pages = (int32_t)v.size();
  for (int i = 0; i < (int)v.size() && i < cap; ++i) out[i] = v[i];
  return ok();
}

int64_t lak_free_pages(const lak_cache* c) { return c ? (int64_t)c->free_list.size() : -1; }

size_t lak_workspace_bytes(const lak_cache* c) { return c ? ws_layout(c).total : 0; }

lak_status lak_kv_append(lak_cache* c, int32_t layer, const void* k_new, const void* v_new, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (c->batch == 0) return ok();
  if (!k_new || !v_new) return fail(LAK_EINVAL, "k_new / v_new is NULL");
  hipError_t e = launch_append(geom(c), c->kp[layer], c->vp[layer], c->d.page_table, c->d.seq_lens, k_new,
                               v_new, c->batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

lak_status lak_kv_prefill(lak_cache* c, int32_t layer, const void* k, const void* v, int64_t t_stride,
                          void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (c->batch == 0) return ok();
  if (!k || !v) return fail(LAK_EINVAL, "k / v is NULL");
  const int mt = c->max_len();
  if (t_stride < mt) return fail(LAK_EINVAL, "t_stride %lld < longest sequence %d", (long long)t_stride, mt);
  hipError_t e = launch_prefill(geom(c), c->kp[layer], c->vp[layer], c->d.page_table, c->d.seq_lens, k, v,
                                t_stride, c->batch, mt, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

lak_status lak_kv_write_rows(lak_cache* c, int32_t layer, int32_t n, const int32_t* rows, const void* k_rows,
                             const void* v_rows, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (n < 0) return fail(LAK_EINVAL, "n < 0");
  if (n > 0 && (!rows || !k_rows)) return fail(LAK_EINVAL, "rows / k_rows is NULL");
  hipError_t e = launch_write_rows(geom(c), c->kp[layer], c->vp[layer], c->d.page_table, c->d.seq_lens, n, rows,
                                   k_rows, v_rows, c->batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "write_rows launch");
  return ok();
}

lak_status lak_kv_gather(lak_cache* c, int32_t layer, int32_t b, int32_t g, int32_t t0, int32_t n, void* k_out,
                         void* v_out, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (b < 0 || b >= c->batch) return fail(LAK_EINVAL, "sequence %d not active", b);
  if (g < 0 || g >= c->d.num_kv_heads) return fail(LAK_EINVAL, "kv head %d out of range", g);
  if (t0 < 0 || n < 0 || (int64_t)t0 + n > c->lens[b])
    return fail(LAK_EINVAL, "tokens [%d, %lld) outside [0, %d)", t0, (long long)t0 + n, c->lens[b]);
  hipError_t e = launch_gather(geom(c), c->kp[layer], c->vp[layer], c->d.page_table, b, g, t0, n, k_out, v_out,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

lak_status lak_kv_gather_scales(lak_cache* c, int32_t layer, int32_t b, int32_t g, int32_t t0, int32_t n,
                                float* k_out, float* v_out, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (c->d.dtype != LAK_FP8_E4M3) return fail(LAK_EINVAL, "only fp8 pools have scales");
  if (b < 0 || b >= c->batch) return fail(LAK_EINVAL, "sequence %d not active", b);
  if (g < 0 || g >= c->d.num_kv_heads) return fail(LAK_EINVAL, "kv head %d out of range", g);
  if (t0 < 0 || n < 0 || (int64_t)t0 + n > c->lens[b])
    return fail(LAK_EINVAL, "tokens [%d, %lld) outside [0, %d)", t0, (long long)t0 + n, c->lens[b]);
  hipError_t e = launch_gather_scales(geom(c), c->kp[layer], c->vp[layer], c->d.page_table, b, g, t0, n, k_out,
                                      v_out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

lak_status lak_attn_full(lak_cache* c, int32_t layer, const void* q, const void* k_new, const void* v_new,
                         float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (c->batch == 0) return ok();
  if (!q || !out) return fail(LAK_EINVAL, "q / out is NULL");
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(LAK_EINVAL, "give both k_new and v_new or neither");
  if ((s = check_ws(c, ws, ws_bytes)) != LAK_OK) return s;
  return run_attention(c, layer, MODE_FULL, q, k_new, v_new, sm_scale, out, lse, nullptr, nullptr, 0, 1, ws,
                       static_cast<hipStream_t>(stream));
}

lak_status lak_attn_delta_select(lak_cache* c, int32_t layer, const void* q, const void* k_new,
                                 const void* v_new, float sm_scale, void* out, float* lse, int32_t k_top,
                                 int32_t recency, int32_t agg, int32_t scope, int32_t* sel, int32_t* sel_count,
                                 int32_t sel_capacity, float* page_scores, void* ws, size_t ws_bytes, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (!q || !out) return fail(LAK_EINVAL, "q / out is NULL");
  if (agg != LAK_AGG_MAX && agg != LAK_AGG_SUM) return fail(LAK_EINVAL, "bad agg %d", agg);
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(LAK_EINVAL, "give both k_new and v_new or neither");
  if ((s = check_select_args(c, scope, k_top, recency, sel, sel_count, sel_capacity)) != LAK_OK) return s;
  if (c->batch == 0) return ok();
  if ((s = check_ws(c, ws, ws_bytes)) != LAK_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  PageScoreArgs pa;
  std::memset(&pa, 0, sizeof(pa));
  s = run_attention(c, layer, MODE_DELTA, q, k_new, v_new, sm_scale, out, lse, nullptr, nullptr, 0, 1, ws, st, agg,
                    &pa.cb);
  if (s != LAK_OK) return s;
  const WsLayout w = ws_layout(c);
  char* wsb = static_cast<char*>(ws);
  float* scores = page_scores ? page_scores : reinterpret_cast<float*>(wsb + w.scores);
  pa.pairs = reinterpret_cast<const float*>(wsb + w.delta);
  pa.rel_blk = reinterpret_cast<const uint8_t*>(wsb + w.delta);
  pa.seq_lens = c->d.seq_lens;
  pa.scores = scores;
  pa.t_pad = (int64_t)c->d.max_pages_per_seq * c->d.page_size;
  pa.hq = c->d.num_q_heads;
  pa.hkv = c->d.num_kv_heads;
  pa.page = c->d.page_size;
  pa.max_pages = c->d.max_pages_per_seq;
  pa.agg = agg;
  pa.scope = scope;
  // score rows x the longest row's tokens: the scoring launch's extent
  pa.tokens_per_block = tune_score_tokens((int64_t)c->batch * (scope == LAK_SCOPE_GROUP ? c->d.num_kv_heads : 1) *
                                          c->max_np() * c->d.page_size);
  const int rows = scope == LAK_SCOPE_GROUP ? c->d.num_kv_heads : 1;
  hipError_t e = launch_delta_post(c->d.dtype, c->d.head_dim, pa, c->batch, rows, c->max_np(), st);
  if (e != hipSuccess) return hip_fail(e, "delta post launch");
  return run_select(c, scores, scope, k_top, recency, sel, sel_count, sel_capacity, st);
}

lak_status lak_page_select(lak_cache* c, const float* page_scores, int32_t scope, int32_t k_top, int32_t recency,
                           int32_t* sel, int32_t* sel_count, int32_t sel_capacity, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if (!page_scores) return fail(LAK_EINVAL, "page_scores is NULL");
  if ((s = check_select_args(c, scope, k_top, recency, sel, sel_count, sel_capacity)) != LAK_OK) return s;
  return run_select(c, page_scores, scope, k_top, recency, sel, sel_count, sel_capacity,
                    static_cast<hipStream_t>(stream));
}

lak_status lak_attn_sparse(lak_cache* c, int32_t layer, const void* q, const void* k_new, const void* v_new,
                           float sm_scale, const int32_t* sel, const int32_t* sel_count, int32_t sel_capacity,
                           int32_t scope, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (c->batch == 0) return ok();
  if (!q || !out) return fail(LAK_EINVAL, "q / out is NULL");
  if (!sel || !sel_count) return fail(LAK_EINVAL, "sel / sel_count is NULL");
  if (sel_capacity <= 0) return fail(LAK_EINVAL, "sel_capacity must be > 0");
  if (scope != LAK_SCOPE_GROUP && scope != LAK_SCOPE_ALL) return fail(LAK_EINVAL, "bad scope %d", scope);
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(LAK_EINVAL, "give both k_new and v_new or neither");
  if ((s = check_ws(c, ws, ws_bytes)) != LAK_OK) return s;
  const int sel_rows = scope == LAK_SCOPE_GROUP ? c->d.num_kv_heads : 1;
  return run_attention(c, layer, MODE_SPARSE, q, k_new, v_new, sm_scale, out, lse, sel, sel_count, sel_capacity,
                       sel_rows, ws, static_cast<hipStream_t>(stream));
}

lak_status lak_attn_sparse_noalloc(lak_cache* c, int32_t layer, const void* q, const void* k_new,
                                   const void* v_new, float sm_scale, const int32_t* sel, const int32_t* sel_count,
                                   int32_t sel_capacity, int32_t scope, void* out, float* lse, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if ((s = check_layer(c, layer)) != LAK_OK) return s;
  if (c->batch == 0) return ok();
  if (!q || !out) return fail(LAK_EINVAL, "q / out is NULL");
  if (!sel || !sel_count) return fail(LAK_EINVAL, "sel / sel_count is NULL");
  if (sel_capacity <= 0) return fail(LAK_EINVAL, "sel_capacity must be > 0");
  if (scope != LAK_SCOPE_GROUP && scope != LAK_SCOPE_ALL) return fail(LAK_EINVAL, "bad scope %d", scope);
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(LAK_EINVAL, "give both k_new and v_new or neither");
  void* parts = nullptr;
  if ((s = noalloc_scratch(&parts)) != LAK_OK) return s;
  const int sel_rows = scope == LAK_SCOPE_GROUP ? c->d.num_kv_heads : 1;
  return run_attention(c, layer, MODE_SPARSE, q, k_new, v_new, sm_scale, out, lse, sel, sel_count, sel_capacity,
                       sel_rows, nullptr, static_cast<hipStream_t>(stream), LAK_AGG_MAX, nullptr, parts,
                       kNoallocScratchBytes);
}

lak_status lak_stack_step(lak_cache* c, const lak_stack_step_desc* st, void* ws, size_t ws_bytes, void* stream) {
  lak_status s = check_cache(c, true);
  if (s != LAK_OK) return s;
  if (!st) return fail(LAK_EINVAL, "step description is NULL");
  const int L = st->num_layers;
  if (L <= 0 || L > c->d.num_layers) return fail(LAK_EINVAL, "num_layers %d outside [1, %d]", L, c->d.num_layers);
  if (!st->tiers || !st->q || !st->k_new || !st->v_new || !st->out || !st->lse || !st->sel || !st->sel_count)
    return fail(LAK_EINVAL, "a per-layer array is NULL");
  if (st->agg != LAK_AGG_MAX && st->agg != LAK_AGG_SUM) return fail(LAK_EINVAL, "bad agg %d", st->agg);
  if ((s = check_ws(c, ws, ws_bytes)) != LAK_OK) return s;
  bool have_sel = false;
  for (int l = 0; l < L; ++l) {
    const int t = st->tiers[l];
    if (t < 0 || t > 2) return fail(LAK_EINVAL, "layer %d: bad tier %d", l, t);
    if ((s = check_layer(c, l)) != LAK_OK) return s;
    if (c->batch > 0 && (!st->q[l] || !st->out[l] || !st->k_new[l] || !st->v_new[l]))
      return fail(LAK_EINVAL, "layer %d: q / out / k_new / v_new is NULL", l);
    if (t == MODE_DELTA) {
      if ((s = check_select_args(c, st->scope, st->k_top, st->recency, st->sel[l], st->sel_count[l],
                                 st->sel_capacity)) != LAK_OK)
        return fail(s, "layer %d: %s", l, g_err.c_str());
      have_sel = true;
    }
    if (t == MODE_SPARSE && !have_sel) return fail(LAK_EINVAL, "sparse layer %d comes before any delta-layer", l);
  }
  if ((s = lak_step_begin(c, stream)) != LAK_OK) return s;
  int cur = -1;
  const hipEvent_t tb0 = c->trace_before, ta0 = c->trace_after;
  for (int l = 0; l < L; ++l) {
    const int t = st->tiers[l];
    if (st->trace_before && st->trace_after) {
      c->trace_before = static_cast<hipEvent_t>(st->trace_before[l]);
      c->trace_after = static_cast<hipEvent_t>(st->trace_after[l]);
      if (!c->trace_before || !c->trace_after) c->trace_before = c->trace_after = nullptr;
    }
    if (t == MODE_FULL) {
      s = lak_attn_full(c, l, st->q[l], st->k_new[l], st->v_new[l], st->sm_scale, st->out[l], st->lse[l], ws,
                        ws_bytes, stream);
    } else if (t == MODE_DELTA) {
      s = lak_attn_delta_select(c, l, st->q[l], st->k_new[l], st->v_new[l], st->sm_scale, st->out[l], st->lse[l],
                                st->k_top, st->recency, st->agg, st->scope, st->sel[l], st->sel_count[l],
                                st->sel_capacity, nullptr, ws, ws_bytes, stream);
      cur = l;
    } else {
      s = lak_attn_sparse(c, l, st->q[l], st->k_new[l], st->v_new[l], st->sm_scale, st->sel[cur], st->sel_count[cur],
                          st->sel_capacity, st->scope, st->out[l], st->lse[l], ws, ws_bytes, stream);
    }
    if (s != LAK_OK) break;
  }
  c->trace_before = tb0;
  c->trace_after = ta0;
  return s == LAK_OK ? ok() : s;
}

lak_status lak_trace_decode(lak_cache* c, void* before, void* after) {
  if (!c) return fail(LAK_EINVAL, "cache is NULL");
  if ((before == nullptr) != (after == nullptr)) return fail(LAK_EINVAL, "set both trace events or neither");
  c->trace_before = static_cast<hipEvent_t>(before);
  c->trace_after = static_cast<hipEvent_t>(after);
  return ok();
}

const char* lak_last_error(void) { return g_err.c_str(); }

}  // extern "C"
