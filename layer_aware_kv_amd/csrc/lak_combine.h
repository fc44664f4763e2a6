// Split-K combine of one (sequence, query head): the weighted sum of the split
// partials, shared by the combine kernel and the delta-layer post kernel.
#pragma once

#include "lak_device.h"
#include "lak_internal.h"

namespace lak {

// Splits holding items of (b, KV head g) for the call described by a.
__device__ inline int combine_splits(const CombineArgs& a, int b, int g) {
  const int T = a.seq_lens[b];
  int n_items;
  if (a.sel_count) {
    const int64_t row = (int64_t)b * a.sel_rows + (a.sel_rows == 1 ? 0 : g);
    n_items = min(max(a.sel_count[row], 0), min(a.sel_cap, (T + a.page - 1) / a.page));
  } else {
    n_items = (T + a.page - 1) / a.page;
  }
  return min((n_items + a.pps - 1) / a.pps, a.splits);
}

// Statistics (M, L) of head h of sequence b over the row's splits (one whole wave).
// With at most 64 splits launched, lane s loads split s's pair together with the row's
// split count (clamped to the launch, skipped past the count); bitwise merge_split_stats.
__device__ inline void head_split_stats(const CombineArgs& a, int b, int h, int lane, float& M, float& L) {
  const float* ml = a.ml_part + ((int64_t)b * a.hq + h) * a.s_cap * 2;
  const int g = h / (a.hq / a.hkv);
  if (a.s_cap >= 1 && a.s_cap <= 64) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = *reinterpret_cast<const f32x2*>(ml + 2 * min(lane, a.s_cap - 1));
    const int S = combine_splits(a, b, g);
    merge_lane_stats(lane < S ? v.x : -INFINITY, v.y, M, L);
  } else {
    merge_split_stats(ml, combine_splits(a, b, g), lane, M, L);
  }
}

// Writes out[b][h] = acc / L (this lane's D/64 elements) and lse[b][h].
template <int ESZ, int D>
__device__ inline void combine_store(const CombineArgs& a, int h, int b, int lane, const float* acc, float M,
                                     float L) {
  constexpr int PER = D / 64;
  const int64_t oi = ((int64_t)b * a.hq + h) * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float val = (L > 0.f) ? acc[e] / L : 0.f;
    if (ESZ == 2)
      reinterpret_cast<uint16_t*>(a.out)[oi + e] = f32_to_bf16_rne(val);
    else
      reinterpret_cast<float*>(a.out)[oi + e] = val;
  }
  if (lane == 0 && a.lse) a.lse[(int64_t)b * a.hq + h] = (L > 0.f) ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// One wave: out[b][h] = sum_s 2^(m_s - M) o_s / L and lse[b][h] = (M + log2 L) ln 2.
// Lane s holds split s's weight; the weighted sum over splits runs in split order with
// the weight broadcast from a scalar register.  Launches of at most NF splits load
// every partial in one round, before the row's split count and statistics are known
// (loads past the launch's split count repeat its last split; splits past the row's
// count are skipped, never multiplied by a zero weight); larger ones (or NF = 0) loop
// over the splits with a group of loads in flight.  Both give the same bits.
template <int ESZ, int D, int NF>
__device__ inline void combine_head(const CombineArgs& a, int h, int b, int lane) {
  constexpr int PER = D / 64;  // head-dim elements per lane
  const int G = a.hq / a.hkv;
  const int64_t row0 = ((int64_t)b * a.hq + h) * a.s_cap;
  float M, L;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  if (NF > 0 && a.s_cap >= 1 && a.s_cap <= NF) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const float* op = a.o_part + row0 * D + lane * PER;
    float v[NF > 0 ? NF : 1][PER];
#pragma unroll
    for (int u = 0; u < NF; ++u) {
      const int uc = min(u, a.s_cap - 1);
#pragma unroll
      for (int e = 0; e < PER; ++e) v[u][e] = op[(int64_t)uc * D + e];
    }
    const f32x2 ml = *reinterpret_cast<const f32x2*>(a.ml_part + (row0 + min(lane, a.s_cap - 1)) * 2);
    const int S = combine_splits(a, b, h / G);
    merge_lane_stats(lane < S ? ml.x : -INFINITY, ml.y, M, L);
    if (M != -INFINITY) {
      const float wl = (lane < S) ? exp2f(ml.x - M) : 0.f;
#pragma unroll
      for (int u = 0; u < NF; ++u) {
        if (u < S) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += w * v[u][e];
        }
      }
    }
    combine_store<ESZ, D>(a, h, b, lane, acc, M, L);
    return;
  }
  const int S = combine_splits(a, b, h / G);
  merge_split_stats(a.ml_part + row0 * 2, S, lane, M, L);
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < S; c0 += 64) {
      const int s_l = c0 + lane;
      const float wl = (s_l < S) ? exp2f(a.ml_part[(row0 + s_l) * 2] - M) : 0.f;
      const int cn = min(64, S - c0);
      const float* op = a.o_part + (row0 + c0) * D + lane * PER;
      int s = 0;
      for (; s + 8 <= cn; s += 8) {
        float v[8][PER];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < PER; ++e) v[u][e] = op[(int64_t)(s + u) * D + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s + u));
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] += w * v[u][e];
        }
      }
      for (; s < cn; ++s) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += w * op[(int64_t)s * D + e];
      }
    }
  }
  combine_store<ESZ, D>(a, h, b, lane, acc, M, L);
}

}  // namespace lak
