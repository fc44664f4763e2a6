// Host-side declarations shared by the ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lak {

enum Mode { MODE_FULL = 0, MODE_DELTA = 1, MODE_SPARSE = 2 };

constexpr size_t kLdsBytesPerCu = 160 * 1024;  // LDS of one gfx950 compute unit

// Arguments of the split-K decode kernel (all three tiers).
struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  const int32_t* page_table;   // [max_batch][max_pages]
  const int32_t* seq_lens;     // [max_batch]
  const void* q;               // [B][Hq][D]
  const void* k_new;           // optional [B][Hkv][D]: token appended at T-1 by this call
  const void* v_new;           // (bfloat16 rows for fp8 pools, encoded by the kernel)
  const float* k_scale;        // fp8 pools: per-token scales [page][Hkv][P] after the codes
  const float* v_scale;
  float sm_scale;
  int hq, hkv, page, max_pages;
  int pps;                     // items (pages or selection entries) per split
  int s_cap;                   // split stride of the partial buffers (= splits launched)
  // sparse tier
  const int32_t* sel;          // [B][R][sel_cap]
  const int32_t* sel_count;    // [B][R]
  int sel_cap;
  int sel_rows;                // R: Hkv (per KV head) or 1 (shared)
  // outputs
  float* o_part;               // [B][Hq][s_cap][D]
  float* ml_part;              // [B][Hq][s_cap][2]  (max in log2 units, sum)
  // delta tier, MAX aggregation: per (b, g, 16-token sub-tile) one block of
  // max_block_bytes(G) bytes: every token's weight relative to the head's sub-tile max r,
  // 2^(logit - r), in fp16 as [G heads][16 tokens], then the G maxima r (float32, log2
  // units); blocks are [B][Hkv][t_pad/16]
  uint8_t* rel_blk;
  int lds_stage;               // delta tier: stage the scratch in LDS, write it at the split's end
  float* pairs;                // delta tier, SUM aggregation: per (head, sub-tile) the pair
  int sum_pairs;               // (max logit in log2 units, sum of 2^(logit - max)) [..][Gp][2]
  int64_t t_pad;               // token capacity of a sequence (max_pages * page)
};

struct CombineArgs {
  const float* o_part;
  const float* ml_part;
  const int32_t* seq_lens;
  const int32_t* sel_count;   // sparse tier: [B][R]; NULL for full
  int sel_cap, sel_rows;
  int hq, hkv, page, pps, s_cap;
  int splits;                 // splits launched by the decode kernel
  void* out;                  // [B][Hq][D]
  float* lse;                 // [B][Hq] (may be NULL)
};

struct PageScoreArgs {
  const uint8_t* rel_blk;     // MAX: the blocks of relative weights and sub-tile maxima as the
                              //      decode kernel wrote them (DecodeArgs::rel_blk)
  const float* pairs;         // SUM: (max, sum) pairs
  CombineArgs cb;             // the delta decode's split partials: each head's LSE is merged
                              // from them, and extra blocks write the layer's out / lse
  const int32_t* seq_lens;
  float* scores;              // [B][R][max_pages]
  int64_t t_pad;
  int hq, hkv, page, max_pages;
  int agg;                    // 0 max, 1 sum
  int scope;                  // 0 group, 1 all
  int tokens_per_block;
};

// Delta-layer post step in one launch: the split combine (out, lse) and the page scores
// (MAX from the fp16 relative weights, SUM from the (max, sum) pairs).
hipError_t launch_delta_post(int dtype, int D, const PageScoreArgs& a, int batch, int rows, int max_np,
                             hipStream_t st);

struct TopkArgs {
  const float* scores;        // [B][R][max_pages]
  const int32_t* seq_lens;
  int32_t* sel;               // [B][R][sel_cap]
  int32_t* sel_count;         // [B][R]
  int rows_per_seq;           // R
  int page, max_pages, k_top, recency, sel_cap;
  int max_np;                 // most pages of any row in the call (host lengths): picks the kernel
};

constexpr int kStepMax = 96;
struct StepUpdate {
  int32_t n;          // page-table entries to write
  int32_t batch;      // sequences whose length grows by one (0: none)
  int32_t b[kStepMax];
  int32_t lp[kStepMax];
  int32_t page[kStepMax];
};

struct KvGeom {
  int hkv, d, page, max_pages, esz;  // esz 1: fp8 codes (bfloat16 rows in and out of the library)
  int64_t scale_off;                 // fp8: byte offset of the [page][Hkv][P] float32 scales in a pool
};

// Tuning knobs, read once from the environment (defaults are the tuned values):
//   LAK_TUNE_DECODE_BATCH  sub-tiles loaded together per wave, full tier (1 or 2)
//   LAK_TUNE_DELTA_BATCH   the same for the delta tier (1 or 2; 0, the default: 2 with fp8
//                          pools where the LDS stage limits a CU to three workgroups, else 1)
//   LAK_TUNE_SPARSE_BATCH  the same for the sparse tier (1, 2 or 4; 0, the default: 2 with
//                          fp8 pools or when a wave's whole share is at most two sub-tiles,
//                          else 1); fp32 pools always take 1
//   LAK_TUNE_TARGET_WGS    workgroups a full split-K launch aims for (default 768)
//   LAK_TUNE_SPARSE_WGS    workgroups a sparse split-K launch aims for (default 1024)
//   LAK_TUNE_DELTA_WGS     workgroups a delta split-K launch aims for (default: the fewest
//                          whose LDS stage fits three per CU where the stage limits
//                          occupancy, else 1536 for long calls and 1024 for short ones)
//   LAK_TUNE_RAGGED_WGS    workgroups a full / delta launch over a ragged batch aims for (3072)
//   LAK_TUNE_DELTA_LDS     1 (default): delta scratch staged in LDS, written at a split's end
//   LAK_TUNE_MIN_SUBTILES  fewest 16-token sub-tiles a split-K workgroup is given (default 8)
//   LAK_TUNE_SCORE_TOKENS  tokens of one score row per MAX page-scoring block (default: 1024
//                          to 4096, as many as keep the launch near 1024 blocks)
//   LAK_TUNE_TOPK_WAVE_KPL  largest candidate row (in 64-page units) that the one-wave
//                          selector takes (0, the default: the workgroup selector always)
int tune_decode_batch(int mode);

// Bytes of one sub-tile's MAX block: G heads x 16 fp16 weights, then G float maxima,
// rounded up to whole 32-byte units (G = 7: 252 -> 256).
__host__ __device__ inline int max_block_bytes(int G) { return (G * (16 * 2 + 4) + 31) & ~31; }

// LDS bytes of a delta split's staged blocks: MAX, one block per sub-tile; SUM, the
// (max, sum) pair per (head, sub-tile), Gp = G rounded up to even heads.
inline size_t delta_stage_bytes(int pps, int page, int G, bool sum = false) {
  const size_t gp = (size_t)(G + (G & 1));
  return (size_t)pps * (page / 16) * (sum ? gp * 2 * 4 : (size_t)max_block_bytes(G));
}
// Workgroups a split-K launch of `mode` aims for; the delta tier's depends on the call's
// total items `work`, the LDS stage bytes per item and the sub-tiles per item.
int tune_target_wgs(int mode, int64_t work, size_t stage_per_item, int subtiles_per_item);
int tune_topk_wave_kpl();
// Tokens of a score row per MAX page-scoring block, for `row_tokens` tokens in all rows.
int tune_score_tokens(int64_t row_tokens);
int tune_ragged_wgs();
int tune_delta_lds();
int tune_min_subtiles();

// launchers (return hipSuccess or the launch error)
// ev0 / ev1 (both or neither): events that take the decode kernel's start and end times
hipError_t launch_decode(int dtype, int mode, int D, const DecodeArgs& a, int splits, int batch,
                         hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_combine(int dtype, int D, const CombineArgs& a, int batch, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, int batch, hipStream_t st);
hipError_t launch_step_update(const StepUpdate& u, int32_t* page_table, int32_t* seq_lens,
                              int max_pages, hipStream_t st);
hipError_t launch_append(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                         const int32_t* lens, const void* kn, const void* vn, int batch,
                         hipStream_t st);
hipError_t launch_prefill(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                          const int32_t* lens, const void* k, const void* v, int64_t t_stride,
                          int batch, int max_t, hipStream_t st);
hipError_t launch_write_rows(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                             const int32_t* lens, int n, const int32_t* rows, const void* kr,
                             const void* vr, int batch, hipStream_t st);
hipError_t launch_gather(const KvGeom& g, const void* kp, const void* vp, const int32_t* pt,
                         int b, int gh, int t0, int n, void* ko, void* vo, hipStream_t st);
hipError_t launch_gather_scales(const KvGeom& g, const void* kp, const void* vp, const int32_t* pt,
                                int b, int gh, int t0, int n, float* ko, float* vo, hipStream_t st);

}  // namespace lak
