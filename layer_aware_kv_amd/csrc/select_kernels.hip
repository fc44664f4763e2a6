// Delta-layer page scoring and page selection ("Methodology in Plain English",
// DELTA AI summary page): per token, the maximum (or sum) over the scope's heads of
// the softmax weight exp(logit - lse); per page, the sum over its valid tokens;
// then the last `recency` pages plus the `k_top` highest-scoring older pages.
#include <math.h>

#include "lak_device.h"
#include "lak_internal.h"

namespace lak {

// One block = `tokens_per_block` consecutive tokens of one score row; each thread
// takes 4 consecutive tokens, so a page of P tokens is P/4 adjacent lanes and its
// sum is a butterfly over them (fixed order: scores are bitwise reproducible).
// Input: the decode kernel's blocks per (b, KV head g, 16-token sub-tile): [Gp heads]
// [16 tokens] fp16 weights u relative to the head's sub-tile max r (log2 units), and
// the maxima [Gp].  Token weight of head h: u * 2^(r - lse_h log2 e), the softmax
// weight exp(logit - lse_h) up to the fp16 rounding of u.
template <int P>
__global__ __launch_bounds__(256) void page_score_kernel(PageScoreArgs a) {
  static_assert(P % 16 == 0 && P / 4 <= 64, "page of 16..256 tokens");
  const int chunk = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int NP = min((T + P - 1) / P, a.max_pages);
  const int t_end = NP * P;
  const int G = a.hq / a.hkv;
  const int Gp = G + (G & 1);
  const int g_lo = a.scope == 0 ? r : 0;
  const int g_hi = a.scope == 0 ? r + 1 : a.hkv;
  const int rows = a.scope == 0 ? a.hkv : 1;
  const int64_t nsub = a.t_pad / 16;
  const float* ls = a.lse + (int64_t)b * a.hq;
  float* out = a.scores + ((int64_t)b * rows + r) * a.max_pages;
  const int tb0 = chunk * a.tokens_per_block;
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
        for (int h = 0; h < G; ++h) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(up + h * 16);
          const float c = exp2f(rp[h] - ls[g * G + h] * kLog2e);
          const float u[4] = {(float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] & 0xFFFFu)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[0] >> 16)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] & 0xFFFFu)),
                              (float)__builtin_bit_cast(_Float16, (uint16_t)(w[1] >> 16))};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = (t + e < T) ? u[e] * c : 0.f;
            acc[e] = (a.agg == 0) ? fmaxf(acc[e], x) : acc[e] + x;
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

hipError_t launch_page_score(const PageScoreArgs& a, int batch, int rows, int max_np,
                             hipStream_t st) {
  if (batch == 0 || max_np == 0) return hipSuccess;
  const int64_t tokens = (int64_t)max_np * a.page;
  dim3 grid((unsigned)((tokens + a.tokens_per_block - 1) / a.tokens_per_block), rows, batch);
  switch (a.page) {
    case 16: hipLaunchKernelGGL(page_score_kernel<16>, grid, dim3(256), 0, st, a); break;
    case 32: hipLaunchKernelGGL(page_score_kernel<32>, grid, dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL(page_score_kernel<64>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// SUM aggregation without logits: one thread per page adds, over the scope's KV
// heads, the page's sub-tiles and the group's heads, e * exp(r ln 2 - lse_h) from the
// (r, e) pairs the delta decode kernel wrote per (b, g, sub-tile, head) -- that is
// sum_t exp(logit_t - lse_h) over the page's valid tokens, exactly.
__global__ __launch_bounds__(256) void page_score_pairs_kernel(PageScoreArgs a) {
  const int r = blockIdx.y, b = blockIdx.z;
  const int jp = blockIdx.x * blockDim.x + threadIdx.x;
  const int T = a.seq_lens[b];
  const int NP = min((T + a.page - 1) / a.page, a.max_pages);
  if (jp >= NP) return;
  const int G = a.hq / a.hkv;
  const int Gp = G + (G & 1);
  const int g_lo = a.scope == 0 ? r : 0;
  const int g_hi = a.scope == 0 ? r + 1 : a.hkv;
  const int rows = a.scope == 0 ? a.hkv : 1;
  const int spp = a.page / 16;
  const int64_t nsub = a.t_pad / 16;
  const float* ls = a.lse + (int64_t)b * a.hq;
  float acc = 0.f;
  for (int g = g_lo; g < g_hi; ++g) {
    for (int u = 0; u < spp; ++u) {
      const int st = jp * spp + u;
      if (st * 16 >= T) break;
      const float* pp = a.pairs + ((((int64_t)b * a.hkv + g) * nsub + st) * Gp) * 2;
      for (int h = 0; h < G; ++h) acc += pp[2 * h + 1] * expf(pp[2 * h] * kLn2 - ls[g * G + h]);
    }
  }
  a.scores[((int64_t)b * rows + r) * a.max_pages + jp] = acc;
}

hipError_t launch_page_score_pairs(const PageScoreArgs& a, int batch, int rows, int max_np, hipStream_t st) {
  if (batch == 0 || max_np == 0) return hipSuccess;
  dim3 grid((unsigned)((max_np + 255) / 256), rows, batch);
  hipLaunchKernelGGL(page_score_pairs_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
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
