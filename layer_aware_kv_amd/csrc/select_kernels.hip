// Delta-layer page scoring and page selection ("Methodology in Plain English",
// DELTA AI summary page): per token, the maximum (or sum) over the scope's heads of
// the softmax weight exp(logit - lse); per page, the sum over its valid tokens;
// then the last `recency` pages plus the `k_top` highest-scoring older pages.
#include <math.h>

#include "lak_device.h"
#include "lak_internal.h"

namespace lak {

// One block = `tokens_per_block` consecutive tokens of one score row; one token per
// thread per pass; the page sum is a butterfly over the P lanes of the page
// (fixed order, so scores are bitwise reproducible).
template <int P>
__global__ __launch_bounds__(256) void page_score_kernel(PageScoreArgs a) {
  const int chunk = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int T = a.seq_lens[b];
  const int NP = min((T + P - 1) / P, a.max_pages);
  const int t_end = NP * P;
  const int G = a.hq / a.hkv;
  const int h0 = a.scope == 0 ? r * G : 0;
  const int nh = a.scope == 0 ? G : a.hq;
  const int rows = a.scope == 0 ? a.hkv : 1;
  const float* lg = a.logits + ((int64_t)b * a.hq + h0) * a.t_pad;
  const float* ls = a.lse + (int64_t)b * a.hq + h0;
  float* out = a.scores + ((int64_t)b * rows + r) * a.max_pages;
  const int tb0 = chunk * a.tokens_per_block;
  const int tb1 = min(tb0 + a.tokens_per_block, t_end);
  for (int base = tb0; base < tb1; base += blockDim.x) {
    const int t = base + threadIdx.x;
    float acc = 0.f;
    if (t < T && t < tb1) {
      for (int hh = 0; hh < nh; ++hh) {
        const float w = expf(lg[(int64_t)hh * a.t_pad + t] - ls[hh]);
        acc = (a.agg == 0) ? fmaxf(acc, w) : acc + w;
      }
    }
#pragma unroll
    for (int o = 1; o < P; o <<= 1) acc += shfl_xor_f(acc, o);
    if ((t % P) == 0 && t < tb1) out[t / P] = acc;
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

// Order key of a score: float32 bits of a positive score (monotone for x >= 0);
// zero, negative and NaN scores all map to 0.
__device__ inline uint32_t score_key(float x) { return (x > 0.f) ? __float_as_uint(x) : 0u; }

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

// One score row per block (256 threads).  Radix select (4 passes of 8 bits, most
// significant first) finds tau, the key of the kk-th largest candidate, and how
// many candidates equal to tau are still needed; those are taken in ascending page
// order (lower index wins ties).  A block-wide scan then writes the selected pages
// (older winners and the recency window) in ascending order.
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  __shared__ int hist[256];
  __shared__ int sh_bin, sh_rem;
  __shared__ int wsum[8];
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

  uint32_t tau = 0;
  int need_eq = 0;
  if (radix) {
    uint32_t prefix = 0, mask = 0;
    int rem = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int jj = tid; jj < NC; jj += blockDim.x) {
        const uint32_t key = score_key(S[jj]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
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
    for (int jj = j0; jj < min(j1, NC); ++jj) eqc += (score_key(S[jj]) == tau);
  int dummy;
  const int eq_base = block_excl_scan(eqc, &dummy, wsum);

  auto flag = [&](int jj, int& eqr) -> bool {
    if (jj >= NC || all_c) return true;
    if (!radix) return false;
    const uint32_t key = score_key(S[jj]);
    if (key > tau) return true;
    if (key == tau) return (eqr++) < need_eq;
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
  hipLaunchKernelGGL(topk_kernel, dim3(a.rows_per_seq, batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lak
