// Delta-layer page scoring and page selection ("Methodology in Plain English",
// DELTA AI summary page): per token, the maximum (or sum) over the scope's heads of
// the softmax weight exp(logit - lse); per page, the sum over its valid tokens;
// then the last `recency` pages plus the `k_top` older pages of largest score.  The
// scoring launch also combines the delta decode's split partials into the layer's
// attention output.
#include <math.h>

#include "lak_combine.h"
#include "lak_device.h"
#include "lak_internal.h"

namespace lak {

// Delta-layer post step, one launch.  Grid (n_chunks + combine blocks, score rows R,
// batch).  Blocks x < n_chunks score pages of row (b, r); the others combine the split
// partials of the row's heads (one head per wave: out and lse of the layer).  A scoring
// block first merges, from the same partials and with the combine's own statistics
// routine (head_split_stats), the log-sum-exp of each head it aggregates.
//
// MAX (SUMP false): a block takes `tokens_per_block` consecutive tokens of its row, 4
// per thread, so a page of P tokens is P/4 adjacent lanes and its sum is a butterfly
// over them (fixed order: scores are bitwise reproducible).  Input: per (b, KV head g,
// 16-token sub-tile) [Gp heads][16 tokens] fp16 weights u relative to the head's
// sub-tile max r (log2 units) and the maxima [Gp]; token weight of head h:
// u * 2^(r - lse2_h) = exp(logit - lse_h) up to the fp16 rounding of u.
// SUM (SUMP true): one thread per page adds, over the scope's KV heads, the page's
// sub-tiles and the group's heads, e * 2^(r - lse2_h) from the (r, e) pairs -- the sum
// of exp(logit - lse_h) over the page's valid tokens.
template <int P, int ESZ, int D, bool SUMP>
__global__ __launch_bounds__(256) void delta_post_kernel(PageScoreArgs a, int n_chunks) {
  static_assert(P % 16 == 0 && P / 4 <= 64, "page of 16..256 tokens");
  extern __shared__ float lse2_s[];  // log-sum-exp (log2 units) of the block's heads
  const int r = blockIdx.y, b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g_lo = a.scope == 0 ? r : 0;
  const int g_hi = a.scope == 0 ? r + 1 : a.hkv;
  const int h_lo = g_lo * G, h_hi = g_hi * G;
  if ((int)blockIdx.x >= n_chunks) {
    const int h = h_lo + 4 * ((int)blockIdx.x - n_chunks) + wave;
    if (h < h_hi) combine_head<ESZ, D, 32>(a.cb, h, b, lane);
    return;
  }
  for (int h = h_lo + wave; h < h_hi; h += 4) {
    float M, L;
    head_split_stats(a.cb, b, h, lane, M, L);
    if (lane == 0) lse2_s[h - h_lo] = (L > 0.f) ? M + log2f(L) : -INFINITY;
  }
  __syncthreads();
  const int T = a.seq_lens[b];
  const int NP = min((T + P - 1) / P, a.max_pages);
  const int Gp = G + (G & 1);
  const int rows = a.scope == 0 ? a.hkv : 1;
  const int64_t nsub = a.t_pad / 16;
  float* out = a.scores + ((int64_t)b * rows + r) * a.max_pages;
  if (SUMP) {
    const int jp = (int)blockIdx.x * blockDim.x + threadIdx.x;
    if (jp >= NP) return;
    const int spp = P / 16;
    float acc = 0.f;
    for (int g = g_lo; g < g_hi; ++g) {
      for (int u = 0; u < spp; ++u) {
        const int st = jp * spp + u;
        if (st * 16 >= T) break;
        const float* pp = a.pairs + ((((int64_t)b * a.hkv + g) * nsub + st) * Gp) * 2;
        for (int h = 0; h < G; ++h) acc += pp[2 * h + 1] * exp2f(pp[2 * h] - lse2_s[g * G + h - h_lo]);
      }
    }
    out[jp] = acc;
    return;
  }
  const int t_end = NP * P;
  const int tb0 = (int)blockIdx.x * a.tokens_per_block;
  const int tb1 = min(tb0 + a.tokens_per_block, t_end);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  for (int base = tb0; base < tb1; base += 4 * blockDim.x) {
    const int t = base + 4 * threadIdx.x;  // first of this thread's 4 tokens
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < tb1) {
      for (int g = g_lo; g < g_hi; ++g) {
        const int64_t blk = ((int64_t)b * a.hkv + g) * nsub + t / 16;
        const uint16_t* up = a.rel_w + blk * Gp * 16 + (t % 16);
        const float* rp = a.rel_max + blk * Gp;
        // every head's weights and maximum are loaded before the first is used (G <= 16)
        u32x2 w[16];
        float rh[16];
#pragma unroll
        for (int h = 0; h < 16; ++h) {
          if (h < G) {
            w[h] = *reinterpret_cast<const u32x2*>(up + h * 16);
            rh[h] = rp[h];
          }
        }
#pragma unroll
        for (int h = 0; h < 16; ++h) {
          if (h < G) {
            const float c = exp2f(rh[h] - lse2_s[g * G + h - h_lo]);
            const float u[4] = {(float)__builtin_bit_cast(_Float16, (uint16_t)(w[h][0] & 0xFFFFu)),
                                (float)__builtin_bit_cast(_Float16, (uint16_t)(w[h][0] >> 16)),
                                (float)__builtin_bit_cast(_Float16, (uint16_t)(w[h][1] & 0xFFFFu)),
                                (float)__builtin_bit_cast(_Float16, (uint16_t)(w[h][1] >> 16))};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaxf(acc[e], (t + e < T) ? u[e] * c : 0.f);
          }
        }
      }
    }
    float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int o = 1; o < P / 4; o <<= 1) sum += shfl_xor_f(sum, o);
    if ((t % P) == 0 && t < tb1) out[t / P] = sum;
  }
}

template <int ESZ, int D, bool SUMP>
static hipError_t launch_delta_post_t(const PageScoreArgs& a, int batch, int rows, int max_np, hipStream_t st) {
  const int G = a.hq / a.hkv;
  const int heads = (rows == 1) ? a.hq : G;  // heads per score row
  const int n_chunks = SUMP ? (max_np + 255) / 256
                            : (int)(((int64_t)max_np * a.page + a.tokens_per_block - 1) / a.tokens_per_block);
  dim3 grid((unsigned)(n_chunks + (heads + 3) / 4), rows, batch);
  const size_t lds = (size_t)heads * sizeof(float);
  switch (a.page) {
    case 16: hipLaunchKernelGGL((delta_post_kernel<16, ESZ, D, SUMP>), grid, dim3(256), lds, st, a, n_chunks); break;
    case 32: hipLaunchKernelGGL((delta_post_kernel<32, ESZ, D, SUMP>), grid, dim3(256), lds, st, a, n_chunks); break;
    case 64: hipLaunchKernelGGL((delta_post_kernel<64, ESZ, D, SUMP>), grid, dim3(256), lds, st, a, n_chunks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int ESZ, int D>
static hipError_t launch_delta_post_d(const PageScoreArgs& a, int batch, int rows, int max_np, hipStream_t st) {
  return a.agg == 1 ? launch_delta_post_t<ESZ, D, true>(a, batch, rows, max_np, st)
                    : launch_delta_post_t<ESZ, D, false>(a, batch, rows, max_np, st);
}

hipError_t launch_delta_post(int dtype, int D, const PageScoreArgs& a, int batch, int rows, int max_np,
                             hipStream_t st) {
  if (batch == 0) return hipSuccess;
  const bool f32 = (dtype == 1);  // outputs: bfloat16 for bf16 and fp8 pools
  if (D == 128) return f32 ? launch_delta_post_d<4, 128>(a, batch, rows, max_np, st)
                           : launch_delta_post_d<2, 128>(a, batch, rows, max_np, st);
  if (D == 64) return f32 ? launch_delta_post_d<4, 64>(a, batch, rows, max_np, st)
                          : launch_delta_post_d<2, 64>(a, batch, rows, max_np, st);
  return hipErrorInvalidValue;
}

// Order key of a score: float32 bits of a positive score (monotone for x >= 0);
// zero, negative and NaN scores all map to 0.
__device__ inline uint32_t score_key(float x) { return (x > 0.f) ? __float_as_uint(x) : 0u; }

// Exclusive prefix sum over the block (blockDim.x a multiple of 64, at most 1024).
__device__ inline int block_excl_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkLdsKeys = 12288;  // rows up to this many pages are staged in LDS (48 KiB)

// One score row per block.  The row's order keys are staged in LDS once (rows
// longer than kTopkLdsKeys are read from global memory instead).  Radix select (4
// passes of 8 bits, most significant first) finds tau, the key of the kk-th
// largest candidate, and how many candidates equal to tau are still needed; those
// are taken in ascending page order (lower index wins ties).  A block-wide scan
// then writes the selected pages (older winners and the recency window) in
// ascending order.
template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds_keys[];
  __shared__ int hist[256];
  __shared__ int sh_bin, sh_rem;
  __shared__ int wsum[kTopkThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.seq_lens[b];
  const int NP = max(0, min((T + a.page - 1) / a.page, a.max_pages));
  const int64_t row = (int64_t)b * a.rows_per_seq + r;
  const float* S = a.scores + row * a.max_pages;
  int32_t* out = a.sel + row * a.sel_cap;
  const int NC = max(0, NP - a.recency);
  const int kk = min(a.k_top, NC);
  const bool all_c = (kk == NC);
  const bool radix = !all_c && kk > 0;

  if (IN_LDS) {
    for (int jj = tid; jj < NC; jj += blockDim.x) lds_keys[jj] = score_key(S[jj]);
    __syncthreads();
  }
  auto key = [&](int jj) -> uint32_t { return IN_LDS ? lds_keys[jj] : score_key(S[jj]); };

  uint32_t tau = 0;
  int need_eq = 0;
  if (radix) {
    uint32_t prefix = 0, mask = 0;
    int rem = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int jj = tid; jj < NC; jj += blockDim.x) {
        const uint32_t k = key(jj);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) {
        int c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) c[q] = hist[4 * lane + q];
        const int tot = c[0] + c[1] + c[2] + c[3];
        int suf = tot;  // sum over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += t;
        }
        int acc = suf - tot;  // candidates in higher bins
#pragma unroll
        for (int q = 3; q >= 0; --q) {
          if (acc < rem && acc + c[q] >= rem) {
            sh_bin = 4 * lane + q;
            sh_rem = rem - acc;
          }
          acc += c[q];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh_bin << shift;
      mask |= 255u << shift;
      rem = sh_rem;
      __syncthreads();
    }
    tau = prefix;
    need_eq = rem;
  }

  const int E = (NP + (int)blockDim.x - 1) / (int)blockDim.x;
  const int j0 = min(tid * E, NP), j1 = min(j0 + E, NP);
  int eqc = 0;
  if (radix)
    for (int jj = j0; jj < min(j1, NC); ++jj) eqc += (key(jj) == tau);
  int dummy;
  const int eq_base = block_excl_scan(eqc, &dummy, wsum);

  auto flag = [&](int jj, int& eqr) -> bool {
    if (jj >= NC || all_c) return true;
    if (!radix) return false;
    const uint32_t k = key(jj);
    if (k > tau) return true;
    if (k == tau) return (eqr++) < need_eq;
    return false;
  };
  int cnt = 0, eqr = eq_base;
  for (int jj = j0; jj < j1; ++jj) cnt += flag(jj, eqr);
  int total;
  int pos = block_excl_scan(cnt, &total, wsum);
  eqr = eq_base;
  for (int jj = j0; jj < j1; ++jj)
    if (flag(jj, eqr)) out[pos++] = jj;
  for (int p = total + tid; p < a.sel_cap; p += blockDim.x) out[p] = -1;
  if (tid == 0) a.sel_count[row] = total;
}

hipError_t launch_topk(const TopkArgs& a, int batch, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  dim3 grid(a.rows_per_seq, batch);
  if (a.max_pages <= kTopkLdsKeys)
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(kTopkThreads), (size_t)a.max_pages * 4, st, a);
  else
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(kTopkThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lak
