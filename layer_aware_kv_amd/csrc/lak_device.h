// Device-side building blocks shared by the kernels: the in-page layout of the
// K/V pools, MFMA fragment types and wave-level reductions (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lak {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;          // waves per decode workgroup
constexpr int kSub = 16;           // tokens per sub-tile (one MFMA N/M dimension)

// ---------------------------------------------------------------------------
// In-page layout.  A page of one KV head holds P tokens as P/16 sub-tiles of
// 16 tokens x D elements.  Inside a sub-tile the elements are ordered so that
// the 64 lanes of a wave fetch MFMA operand fragments with one contiguous
// 1 KiB load per instruction (16 bytes per lane, lane-ordered):
//   K: [D/W][16 tokens][W]                   W = 16 bytes / element size
//      -> lane l, load i: token l%16, elements d = (4i + l/16)*W .. +W
//         (the A operand of the q.K^T MFMA: rows = tokens, k = head dim)
//   V: [D/(16H)][4][16][H][4]                H = W / 4
//      -> lane l, load i: d = 16(H i + h) + l%16 for h < H, tokens 4(l/16) .. +4
//         (the A operand of the P.V MFMA: rows = head dim, k = tokens)
// ---------------------------------------------------------------------------
template <int ESZ>
__host__ __device__ inline int k_off(int tt, int d) {
  constexpr int W = 16 / ESZ;
  return ((d / W) * kSub + tt) * W + d % W;
}
template <int ESZ>
__host__ __device__ inline int v_off(int tt, int d) {
  constexpr int H = (16 / ESZ) / 4;
  return (((d / (16 * H)) * 4 + tt / 4) * 16 + d % 16) * (4 * H) + ((d / 16) % H) * 4 + tt % 4;
}

// fp8 pools (esz 1) use the same formulas with W = 16 codes per lane and H = 4;
// their per-token float32 scales follow all pages' codes as [page][Hkv][P].

// Element offset of (physical page, kv head, token-in-page) sub-tile start.
__device__ inline int64_t subtile_base(int64_t phys, int g, int t_in_page, int hkv, int P, int D) {
  return ((phys * hkv + g) * P + (t_in_page / kSub) * kSub) * (int64_t)D;
}

// ---------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------
__device__ inline float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Pairwise combine with the lane 16 (or 32) apart, in registers: v_permlane16_swap /
// v_permlane32_swap (gfx950) leave lane l holding {v_l, v_(l^16)} (or ^32) across
// their two results, so no LDS crossbar round trip is needed.  Max and add are
// commutative, so the result equals v op shfl_xor(v, 16 or 32) bit for bit.
__device__ inline float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor16_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)((b >> 16) | ((b & 0xFFFF) ? 0x40 : 0));
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// ---------------------------------------------------------------------------
// fp8 rows: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// largest magnitude 448) with one float32 scale per row of D values:
// scale = max|x| / 448, code = round-to-nearest-even(x / scale) after clamping to
// +-448; a row whose scale is 0 gets codes 0.
// ---------------------------------------------------------------------------
constexpr float kE4m3Max = 448.0f;

__device__ inline float e4m3_row_scale(float amax) { return amax / kE4m3Max; }

// Codes of x0 / scale and x1 / scale in the low two bytes (x0 in byte 0).
__device__ inline uint32_t e4m3_encode2(float x0, float x1, float scale) {
  if (!(scale > 0.f)) return 0u;
  const float a = fminf(fmaxf(x0 / scale, -kE4m3Max), kE4m3Max);
  const float b = fminf(fmaxf(x1 / scale, -kE4m3Max), kE4m3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Wave-wide maximum (64 lanes).
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Row scale of a bfloat16 row of d values taken by one whole wave (every lane
// calls it; the maximum is order-independent, so every caller gets the same bits).
__device__ inline float e4m3_wave_row_scale(const uint16_t* row, int d, int lane) {
  float m = 0.f;
  for (int i = lane; i < d; i += 64) m = fmaxf(m, fabsf(bf16_to_f32(row[i])));
  return e4m3_row_scale(wave_max(m));
}

// One wave encodes token tt's K row and V row (d bfloat16 values each; vr may be
// NULL) into the fp8 sub-tiles at kb / vb and stores the scales at *ks / *vs.
__device__ inline void encode_rows_fp8(int d, uint8_t* kb, uint8_t* vb, int tt, float* ks, float* vs,
                                       const uint16_t* kr, const uint16_t* vr, int lane) {
  const float ksc = e4m3_wave_row_scale(kr, d, lane);
  const float vsc = vr ? e4m3_wave_row_scale(vr, d, lane) : 0.f;
  for (int i = lane; i < d; i += 64) {
    kb[k_off<1>(tt, i)] = (uint8_t)(e4m3_encode2(bf16_to_f32(kr[i]), 0.f, ksc) & 0xFFu);
    if (vr) vb[v_off<1>(tt, i)] = (uint8_t)(e4m3_encode2(bf16_to_f32(vr[i]), 0.f, vsc) & 0xFFu);
  }
  if (lane == 0) {
    *ks = ksc;
    if (vr) *vs = vsc;
  }
}

// Statistics of one (row, head) over its S split partials ml[s] = (max in log2 units,
// sum of 2^(logit - max)): M = max_s m_s and L = sum_s l_s 2^(m_s - M).  One whole wave;
// lane s takes splits s, s + 64, ...; the fixed order gives every caller the same bits.
__device__ inline void merge_split_stats(const float* ml, int S, int lane, float& M, float& L) {
  float m = -INFINITY;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, ml[2 * s]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float acc = 0.f;
  if (m != -INFINITY) {
    for (int s = lane; s < S; s += 64) acc += exp2f(ml[2 * s] - m) * ml[2 * s + 1];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  }
  M = m;
  L = acc;
}

// The same statistics when each lane holds at most one split: (m, l) of split `lane`,
// m = -inf on lanes without one.  For S <= 64 this is bitwise merge_split_stats.
__device__ inline void merge_lane_stats(float m_lane, float l_lane, float& M, float& L) {
  float m = m_lane;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float acc = 0.f;
  if (m != -INFINITY) {
    if (m_lane != -INFINITY) acc += exp2f(m_lane - m) * l_lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  }
  M = m;
  L = acc;
}

// Inclusive prefix sum over a wave (64 lanes).
__device__ inline int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

}  // namespace lak
