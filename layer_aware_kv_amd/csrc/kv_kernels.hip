// Paged KV cache maintenance: decode-step page-table update, per-step append,
// bulk prefill, single-row overwrite and logical read-back.  The pages keep the
// whole KV history resident (DELTA evicts nothing: "Methodology in Plain
// English" on the DELTA AI summary page); these kernels only place elements.
#include "lak_device.h"
#include "lak_internal.h"

namespace lak {

__global__ void step_update_kernel(StepUpdate u, int32_t* page_table, int32_t* seq_lens,
                                   int max_pages) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < u.n) page_table[(int64_t)u.b[i] * max_pages + u.lp[i]] = u.page[i];
  if (i < u.batch) seq_lens[i] += 1;
}

hipError_t launch_step_update(const StepUpdate& u, int32_t* page_table, int32_t* seq_lens,
                              int max_pages, hipStream_t st) {
  const int n = u.n > u.batch ? u.n : u.batch;
  if (n == 0) return hipSuccess;
  const int blocks = (n + 255) / 256;
  hipLaunchKernelGGL(step_update_kernel, dim3(blocks), dim3(256), 0, st, u, page_table, seq_lens,
                     max_pages);
  return hipGetLastError();
}

// One (b, kv head) per block: the token at position seq_lens[b] - 1.
template <typename E>
__global__ void append_kernel(KvGeom g, E* kp, E* vp, const int32_t* pt, const int32_t* lens,
                              const E* kn, const E* vn) {
  const int gh = blockIdx.x, b = blockIdx.y;
  const int T = lens[b];
  if (T <= 0) return;
  const int t = T - 1;
  const int lp = t / g.page;
  if (lp >= g.max_pages) return;
  const int64_t phys = pt[(int64_t)b * g.max_pages + lp];
  const int64_t base = subtile_base(phys, gh, t % g.page, g.hkv, g.page, g.d);
  const int tt = t % kSub;
  const int64_t src = ((int64_t)b * g.hkv + gh) * g.d;
  for (int d = threadIdx.x; d < g.d; d += blockDim.x) {
    kp[base + k_off<sizeof(E)>(tt, d)] = kn[src + d];
    vp[base + v_off<sizeof(E)>(tt, d)] = vn[src + d];
  }
}

// One 16-token sub-tile of one (b, kv head) per block: stage the logical rows in
// LDS, then write 16-byte chunks in the pool's sub-tile order.
template <typename E>
__global__ void prefill_kernel(KvGeom g, E* kp, E* vp, const int32_t* pt, const int32_t* lens,
                               const E* ks, const E* vs, int64_t t_stride) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* sk = reinterpret_cast<E*>(smem);
  E* sv = sk + kSub * g.d;
  const int st = blockIdx.x, gh = blockIdx.y, b = blockIdx.z;
  const int T = lens[b];
  const int t0 = st * kSub;
  if (t0 >= T) return;
  const int lp = t0 / g.page;
  const int64_t phys = pt[(int64_t)b * g.max_pages + lp];
  const int64_t base = subtile_base(phys, gh, t0 % g.page, g.hkv, g.page, g.d);
  const int64_t src = (((int64_t)b * g.hkv + gh) * t_stride + t0) * g.d;
  const int n = kSub * g.d;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int tt = i / g.d;
    const bool ok = t0 + tt < T;
    sk[i] = ok ? ks[src + i] : (E)0;
    sv[i] = ok ? vs[src + i] : (E)0;
  }
  __syncthreads();
  constexpr int W = 16 / sizeof(E);
  constexpr int H = W / 4;
  const int nchunk = n / W;
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
    // K chunk c: (d-chunk c/16, token c%16), W contiguous elements
    E kb[W], vb[W];
    const int kt = c % kSub, kd = (c / kSub) * W;
#pragma unroll
    for (int x = 0; x < W; ++x) kb[x] = sk[kt * g.d + kd + x];
    // V chunk c = (p*4 + j)*16 + i: elements [h*4 + e] = V[4j + e][16(H p + h) + i]
    const int vi = c % 16, vj = (c / 16) % 4, vp_ = c / 64;
#pragma unroll
    for (int x = 0; x < W; ++x) {
      const int h = x / 4, e = x % 4;
      vb[x] = sv[(4 * vj + e) * g.d + 16 * (H * vp_ + h) + vi];
    }
    *reinterpret_cast<u32x4*>(kp + base + (int64_t)c * W) = *reinterpret_cast<const u32x4*>(kb);
    *reinterpret_cast<u32x4*>(vp + base + (int64_t)c * W) = *reinterpret_cast<const u32x4*>(vb);
  }
}

template <typename E>
__global__ void write_rows_kernel(KvGeom g, E* kp, E* vp, const int32_t* pt, const int32_t* lens,
                                  int batch, const int32_t* rows, const E* kr, const E* vr) {
  const int r = blockIdx.x;
  const int b = rows[3 * r], gh = rows[3 * r + 1], t = rows[3 * r + 2];
  if (b < 0 || b >= batch || gh < 0 || gh >= g.hkv || t < 0 || t >= lens[b]) return;
  const int lp = t / g.page;
  if (lp >= g.max_pages) return;
  const int64_t phys = pt[(int64_t)b * g.max_pages + lp];
  const int64_t base = subtile_base(phys, gh, t % g.page, g.hkv, g.page, g.d);
  const int tt = t % kSub;
  for (int d = threadIdx.x; d < g.d; d += blockDim.x) {
    kp[base + k_off<sizeof(E)>(tt, d)] = kr[(int64_t)r * g.d + d];
    if (vr) vp[base + v_off<sizeof(E)>(tt, d)] = vr[(int64_t)r * g.d + d];
  }
}

template <typename E>
__global__ void gather_kernel(KvGeom g, const E* kp, const E* vp, const int32_t* pt, int b, int gh,
                              int t0, int n, E* ko, E* vo) {
  const int i = blockIdx.x;  // token
  if (i >= n) return;
  const int t = t0 + i;
  const int lp = t / g.page;
  const int64_t phys = pt[(int64_t)b * g.max_pages + lp];
  const int64_t base = subtile_base(phys, gh, t % g.page, g.hkv, g.page, g.d);
  const int tt = t % kSub;
  for (int d = threadIdx.x; d < g.d; d += blockDim.x) {
    if (ko) ko[(int64_t)i * g.d + d] = kp[base + k_off<sizeof(E)>(tt, d)];
    if (vo) vo[(int64_t)i * g.d + d] = vp[base + v_off<sizeof(E)>(tt, d)];
  }
}

hipError_t launch_append(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                         const int32_t* lens, const void* kn, const void* vn, int batch,
                         hipStream_t st) {
  if (batch == 0) return hipSuccess;
  dim3 grid(g.hkv, batch);
  if (g.esz == 2)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(64), 0, st, g, (uint16_t*)kp,
                       (uint16_t*)vp, pt, lens, (const uint16_t*)kn, (const uint16_t*)vn);
  else
    hipLaunchKernelGGL(append_kernel<uint32_t>, grid, dim3(64), 0, st, g, (uint32_t*)kp,
                       (uint32_t*)vp, pt, lens, (const uint32_t*)kn, (const uint32_t*)vn);
  return hipGetLastError();
}

hipError_t launch_prefill(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                          const int32_t* lens, const void* k, const void* v, int64_t t_stride,
                          int batch, int max_t, hipStream_t st) {
  if (batch == 0 || max_t == 0) return hipSuccess;
  dim3 grid((max_t + kSub - 1) / kSub, g.hkv, batch);
  const size_t lds = 2 * (size_t)kSub * g.d * g.esz;
  if (g.esz == 2)
    hipLaunchKernelGGL(prefill_kernel<uint16_t>, grid, dim3(256), lds, st, g, (uint16_t*)kp,
                       (uint16_t*)vp, pt, lens, (const uint16_t*)k, (const uint16_t*)v, t_stride);
  else
    hipLaunchKernelGGL(prefill_kernel<uint32_t>, grid, dim3(256), lds, st, g, (uint32_t*)kp,
                       (uint32_t*)vp, pt, lens, (const uint32_t*)k, (const uint32_t*)v, t_stride);
  return hipGetLastError();
}

hipError_t launch_write_rows(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                             const int32_t* lens, int n, const int32_t* rows, const void* kr,
                             const void* vr, int batch, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (g.esz == 2)
    hipLaunchKernelGGL(write_rows_kernel<uint16_t>, dim3(n), dim3(64), 0, st, g, (uint16_t*)kp,
                       (uint16_t*)vp, pt, lens, batch, rows, (const uint16_t*)kr,
                       (const uint16_t*)vr);
  else
    hipLaunchKernelGGL(write_rows_kernel<uint32_t>, dim3(n), dim3(64), 0, st, g, (uint32_t*)kp,
                       (uint32_t*)vp, pt, lens, batch, rows, (const uint32_t*)kr,
                       (const uint32_t*)vr);
  return hipGetLastError();
}

hipError_t launch_gather(const KvGeom& g, const void* kp, const void* vp, const int32_t* pt, int b,
                         int gh, int t0, int n, void* ko, void* vo, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (g.esz == 2)
    hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(n), dim3(64), 0, st, g, (const uint16_t*)kp,
                       (const uint16_t*)vp, pt, b, gh, t0, n, (uint16_t*)ko, (uint16_t*)vo);
  else
    hipLaunchKernelGGL(gather_kernel<uint32_t>, dim3(n), dim3(64), 0, st, g, (const uint32_t*)kp,
                       (const uint32_t*)vp, pt, b, gh, t0, n, (uint32_t*)ko, (uint32_t*)vo);
  return hipGetLastError();
}

}  // namespace lak
