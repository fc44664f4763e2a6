// Delta-layer page scoring and page selection ("Methodology in Plain English",
// DELTA AI summary page): per token, the maximum (or sum) over the scope's heads of
// the softmax weight exp(logit - lse); per page, the sum over its valid tokens;
// then the last `recency` pages plus the `k_top` older pages of largest score.  The
// scoring launch also combines the delta decode's split partials into the layer's
// attention output.
#include <math.h>

#include <algorithm>

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
// 16-token sub-tile) one block of [G heads][16 tokens] fp16 weights u relative to the
// head's sub-tile max r (log2 units), then the G maxima; token weight of head h:
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
      const int blk_bytes = max_block_bytes(G);
      for (int g = g_lo; g < g_hi; ++g) {
        const int64_t blk = ((int64_t)b * a.hkv + g) * nsub + t / 16;
        const uint8_t* bp = a.rel_blk + blk * blk_bytes;
        const uint16_t* up = reinterpret_cast<const uint16_t*>(bp) + (t % 16);
        const float* rp = reinterpret_cast<const float*>(bp + G * 32);
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


__device__ inline uint32_t wave_or_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v |= (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}
__device__ inline uint32_t wave_and_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v &= (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}
// popcount of the bits of m below this lane
__device__ inline int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkLdsKeys = 12288;  // rows up to this many pages are staged in LDS (48 KiB)

// One score row per block.  The row's candidate order keys are staged in LDS once
// (rows longer than kTopkLdsKeys are read from global memory instead).  A radix select
// finds the key of the kk-th largest candidate: its digits (8 bits, most significant
// first, counted in an LDS histogram) start at the highest bit in which the row's
// candidates differ (the bits above are common to all of them), and it stops as soon
// as the digit's bin holds exactly the candidates still needed.  One block scan of
// each thread's (larger, equal) counts then places the winners: a thread's first
// output slot is the larger candidates before it plus min(still needed, equal
// candidates before it), so candidates equal to the boundary are taken in page order
// until the count is reached.  The recency window follows every candidate.
template <bool IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ uint32_t lds_keys[];
  __shared__ int hist[256];
  __shared__ int sh_bin, sh_rem, sh_cnt;
  __shared__ uint32_t red_or[kTopkThreads / 64], red_and[kTopkThreads / 64];
  __shared__ int wsum_g[kTopkThreads / 64], wsum_e[kTopkThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (int)blockDim.x >> 6;
  const int T = a.seq_lens[b];
  const int NP = max(0, min((T + a.page - 1) / a.page, a.max_pages));
  const int64_t row = (int64_t)b * a.rows_per_seq + r;
  const float* S = a.scores + row * a.max_pages;
  int32_t* out = a.sel + row * a.sel_cap;
  const int NC = max(0, NP - a.recency);
  const int kk = min(a.k_top, NC);
  const bool all_c = (kk == NC);
  const bool radix = !all_c && kk > 0;

  if (IN_LDS && radix) {
    for (int jj = tid; jj < NC; jj += blockDim.x) lds_keys[jj] = score_key(S[jj]);
    __syncthreads();
  }
  auto key = [&](int jj) -> uint32_t { return IN_LDS ? lds_keys[jj] : score_key(S[jj]); };

  uint32_t prefix = 0, mask = 0;  // the boundary key's known top bits, and which bits those are
  int need = kk;                  // candidates still to take among keys matching prefix on mask
  if (radix) {
    uint32_t kor = 0u, kand = ~0u;
    for (int jj = tid; jj < NC; jj += blockDim.x) {
      const uint32_t k = key(jj);
      kor |= k;
      kand &= k;
    }
    kor = wave_or_u32(kor);
    kand = wave_and_u32(kand);
    if (lane == 0) {
      red_or[wave] = kor;
      red_and[wave] = kand;
    }
    __syncthreads();
    kor = 0u;
    kand = ~0u;
    for (int w = 0; w < nw; ++w) {
      kor |= red_or[w];
      kand &= red_and[w];
    }
    const uint32_t diff = kor & ~kand;  // bits in which some candidates differ
    if (diff == 0u) {
      prefix = kand;  // all candidates equal: the first kk in page order
      mask = ~0u;
    } else {
      const int hb = 31 - __builtin_clz(diff);  // <= 30: keys of scores are at most 0x7F800000
      mask = ~0u << (hb + 1);
      prefix = kand & mask;
      for (int top = hb; top >= 0; top -= 8) {
        const int shift = max(top - 7, 0);
        const uint32_t dmask = (1u << (top - shift + 1)) - 1u;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int jj = tid; jj < NC; jj += blockDim.x) {
          const uint32_t k = key(jj);
          if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
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
            if (acc < need && acc + c[q] >= need) {
              sh_bin = 4 * lane + q;
              sh_rem = need - acc;
              sh_cnt = c[q];
            }
            acc += c[q];
          }
        }
        __syncthreads();
        // every thread reads these before wave 0 can write them again (two barriers later)
        prefix |= (uint32_t)sh_bin << shift;
        mask |= dmask << shift;
        need = sh_rem;
        if (sh_cnt == need) break;  // the whole bin is taken: lower digits cannot change the choice
      }
    }
  }

  // each thread takes E consecutive candidates
  const int E = (NC + (int)blockDim.x - 1) / (int)blockDim.x;
  const int j0 = min(tid * E, NC), j1 = min(j0 + E, NC);
  int gt = 0, eq = 0;
  if (all_c) {
    gt = j1 - j0;
  } else if (radix) {
    for (int jj = j0; jj < j1; ++jj) {
      const uint32_t km = key(jj) & mask;
      gt += km > prefix;
      eq += km == prefix;
    }
  }
  const int gt_inc = wave_incl_scan(gt, lane), eq_inc = wave_incl_scan(eq, lane);
  if (lane == 63) {
    wsum_g[wave] = gt_inc;
    wsum_e[wave] = eq_inc;
  }
  __syncthreads();
  int gt_before = gt_inc - gt, eq_before = eq_inc - eq;
  for (int w = 0; w < wave; ++w) {
    gt_before += wsum_g[w];
    eq_before += wsum_e[w];
  }
  int pos = gt_before + min(need, eq_before);
  int eqr = eq_before;
  for (int jj = j0; jj < j1; ++jj) {
    bool take = all_c;
    if (radix) {
      const uint32_t km = key(jj) & mask;
      take = km > prefix || (km == prefix && eqr++ < need);
    }
    if (take) out[pos++] = jj;
  }
  const int nrec = NP - NC;  // the recency window, after every candidate
  for (int q = tid; q < nrec; q += blockDim.x) out[kk + q] = NC + q;
  const int total = kk + nrec;
  for (int p = total + tid; p < a.sel_cap; p += blockDim.x) out[p] = -1;
  if (tid == 0) a.sel_count[row] = total;
}

// One wave per score row: the same selection as topk_kernel with no workgroup
// barrier.  Lane l holds the order keys of candidate pages 64 i + l (i < KPL) in
// registers.  The kk-th largest candidate key is found by a radix select whose first
// digit starts at the highest bit in which the row's candidate keys differ (the bits
// above are common to all of them).  Each digit of up to 6 bits is counted in LDS in
// per-lane histograms (lane l adds only to its own 64 counters, so no two lanes ever
// add to the same word), summed across lanes by 64 lanes reading one bin each; the
// select stops as soon as the digit's bin holds exactly the keys still needed.  The
// chosen candidates are then written in ascending order, 64 at a time, at offsets
// from wave ballots (candidates equal to the boundary key are taken in page order
// until the count is reached), and the recency pages after them.
constexpr int kWaveBins = 64;         // 6-bit digits
constexpr int kWaveHistStride = 65;   // words per lane: lane l's counter b sits in bank (l + b) mod 32

template <int KPL>
__global__ __launch_bounds__(64) void topk_wave_kernel(TopkArgs a) {
  __shared__ int hist[64 * kWaveHistStride];
  const int r = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int T = a.seq_lens[b];
  const int NP = max(0, min((T + a.page - 1) / a.page, a.max_pages));
  const int64_t row = (int64_t)b * a.rows_per_seq + r;
  const float* S = a.scores + row * a.max_pages;
  int32_t* out = a.sel + row * a.sel_cap;
  // candidates beyond 64 * KPL are never looked at (the host picks KPL from the call's lengths)
  const int NC = min(max(0, NP - a.recency), 64 * KPL);
  const int kk = min(a.k_top, NC);
  const bool all_c = (kk == NC);
  const bool radix = !all_c && kk > 0;

  // Candidates' keys are at most 0x7F800000; other slots hold kNotCand, whose top bit no
  // candidate shares, so they never match a prefix of the candidates.  Every load is
  // issued unconditionally, clamped into the row (always in bounds: the row holds
  // max_pages >= 1 entries), so that no per-register condition stays live.
  constexpr uint32_t kNotCand = 0xFFFFFFFFu;
  uint32_t key[KPL];
  const int jmax = max(NC - 1, 0);
#pragma unroll
  for (int i = 0; i < KPL; ++i) key[i] = __float_as_uint(S[min(64 * i + lane, jmax)]);
#pragma unroll
  for (int i = 0; i < KPL; ++i)
    key[i] = (64 * i + lane < NC) ? (radix ? score_key(__uint_as_float(key[i])) : 0u) : kNotCand;

  uint32_t prefix = 0, mask = 0;  // the boundary key's known top bits, and which bits those are
  int need = kk;                  // candidates still to take among keys matching prefix on mask
  if (radix) {
    uint32_t kor = 0u, kand = ~0u;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      kor |= (key[i] == kNotCand) ? 0u : key[i];
      kand &= key[i];
    }
    kor = wave_or_u32(kor);
    kand = wave_and_u32(kand);
    const uint32_t diff = kor & ~kand;  // bits in which some candidates differ
    if (diff == 0u) {
      prefix = kand;  // all candidates equal: the first kk in page order
      mask = ~0u;
    } else {
      const int hb = 31 - __builtin_clz(diff);  // <= 30: candidates' top bit is 0
      mask = ~0u << (hb + 1);
      prefix = kand & mask;
      int* mine = hist + lane * kWaveHistStride;
      for (int q = 0; q < kWaveBins; ++q) mine[q] = 0;
      for (int top = hb; top >= 0; top -= 6) {
        const int shift = max(top - 5, 0);
        const uint32_t dmask = (1u << (top - shift + 1)) - 1u;
#pragma unroll
        for (int i = 0; i < KPL; ++i)
          if ((key[i] & mask) == prefix) atomicAdd(mine + ((key[i] >> shift) & dmask), 1);
        __syncthreads();
        // lane q sums bin q over the 64 lanes' histograms and clears them for the next digit
        int c = 0;
#pragma unroll 8
        for (int l2 = 0; l2 < 64; ++l2) {
          c += hist[l2 * kWaveHistStride + lane];
          hist[l2 * kWaveHistStride + lane] = 0;
        }
        // higher bins hold larger keys: acc = candidates in the bins above this lane's
        int suf = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += t;
        }
        const int acc = suf - c;
        const bool here = acc < need && acc + c >= need;
        const unsigned long long won = __ballot(here);
        const int src = __ffsll(won) - 1;  // exactly one lane holds the boundary bin
        const int rem = __shfl(need - acc, src, 64);
        const int cnt = __shfl(c, src, 64);
        prefix |= (uint32_t)src << shift;
        mask |= dmask << shift;
        need = rem;
        __syncthreads();  // the cleared counters are in place before the next digit's adds
        if (cnt == rem) break;  // the whole bin is taken: lower digits cannot change the choice
      }
    }
  }

  // candidates in page order, then the recency window (always after every candidate)
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    if (64 * i >= NC) break;
    const int j = 64 * i + lane;
    const bool cand = key[i] != kNotCand;  // j < NC (recomputing it would keep KPL masks live)
    const bool eq = radix && (key[i] & mask) == prefix;  // never for kNotCand
    const unsigned long long eqm = __ballot(eq);
    const int eq_rank = eq_seen + lanes_below(eqm);
    eq_seen += __popcll(eqm);
    const bool take = cand && (all_c || (radix && ((key[i] & mask) > prefix || (eq && eq_rank < need))));
    const unsigned long long tm = __ballot(take);
    if (take) out[base + lanes_below(tm)] = j;
    base += __popcll(tm);
  }
  const int nrec = NP - max(0, NP - a.recency);
  for (int q = lane; q < nrec; q += 64) out[base + q] = NP - nrec + q;
  base += nrec;
  for (int p = base + lane; p < a.sel_cap; p += 64) out[p] = -1;
  if (lane == 0) a.sel_count[row] = base;
}

constexpr int kWaveTopkMaxKpl = 128;  // up to 8192 candidate pages per row take the one-wave selector

hipError_t launch_topk(const TopkArgs& a, int batch, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  dim3 grid(a.rows_per_seq, batch);
  const int kpl = (std::max(a.max_np - a.recency, 0) + 63) / 64;
  const int wave_max = std::min(kWaveTopkMaxKpl, tune_topk_wave_kpl());
  if (wave_max > 0 && kpl <= wave_max) {
    if (kpl <= 16) hipLaunchKernelGGL(topk_wave_kernel<16>, grid, dim3(64), 0, st, a);
    else if (kpl <= 32) hipLaunchKernelGGL(topk_wave_kernel<32>, grid, dim3(64), 0, st, a);
    else if (kpl <= 64) hipLaunchKernelGGL(topk_wave_kernel<64>, grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL(topk_wave_kernel<128>, grid, dim3(64), 0, st, a);
  } else if (a.max_pages <= kTopkLdsKeys) {
    hipLaunchKernelGGL(topk_kernel<true>, grid, dim3(kTopkThreads), (size_t)a.max_pages * 4, st, a);
  } else {
    hipLaunchKernelGGL(topk_kernel<false>, grid, dim3(kTopkThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace lak
