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

// One wave: out[b][h] = sum_s 2^(m_s - M) o_s / L and lse[b][h] = (M + log2 L) ln 2.
// Lane s holds split s's weight; the weighted sum over splits runs in split order with
// the weight broadcast from a scalar register and an unrolled group of split loads
// in flight together.
template <int ESZ, int D>
__device__ inline void combine_head(const CombineArgs& a, int h, int b, int lane) {
  constexpr int PER = D / 64;  // head-dim elements per lane
  const int G = a.hq / a.hkv;
  const int S = combine_splits(a, b, h / G);
  const int64_t row0 = ((int64_t)b * a.hq + h) * a.s_cap;
  float M, L;
  merge_split_stats(a.ml_part + row0 * 2, S, lane, M, L);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
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

}  // namespace lak
