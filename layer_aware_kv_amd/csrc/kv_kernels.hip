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


// ---------------------------------------------------------------------------
// fp8 pools: rows arrive as bfloat16 and are stored as E4M3 codes plus one
// float32 scale per (token, KV head) row (see e4m3_encode2).
// ---------------------------------------------------------------------------
__device__ inline float* scale_ptr(uint8_t* pool, const KvGeom& g) {
  return reinterpret_cast<float*>(pool + g.scale_off);
}

// One wave encodes one K row and one V row of D bfloat16 values into the sub-tile
// at `base` (token tt of the sub-tile) and stores their scales at scale index si.
__device__ inline void encode_row_fp8(const KvGeom& g, uint8_t* kp, uint8_t* vp, int64_t base, int tt,
                                      int64_t si, const uint16_t* kr, const uint16_t* vr, int lane) {
  encode_rows_fp8(g.d, kp + base, vp + base, tt, scale_ptr(kp, g) + si, scale_ptr(vp, g) + si, kr, vr, lane);
}

__global__ void append_fp8_kernel(KvGeom g, uint8_t* kp, uint8_t* vp, const int32_t* pt, const int32_t* lens,
                                  const uint16_t* kn, const uint16_t* vn) {
  const int gh = blockIdx.x, b = blockIdx.y;
  const int T = lens[b];
  if (T <= 0) return;
  const int t = T - 1;
  const int lp = t / g.page;
  if (lp >= g.max_pages) return;
  const int64_t phys = pt[(int64_t)b * g.max_pages + lp];
  const int64_t base = subtile_base(phys, gh, t % g.page, g.hkv, g.page, g.d);
  const int64_t src = ((int64_t)b * g.hkv + gh) * g.d;
  encode_row_fp8(g, kp, vp, base, t % kSub, (phys * g.hkv + gh) * g.page + t % g.page, kn + src, vn + src,
                 threadIdx.x);
}

// One 16-token sub-tile of one (b, kv head) per block of 256 threads: stage the 16
// K and 16 V rows in LDS, take each row's scale (8 threads per row), then write
// 16-byte chunks of codes in the sub-tile order and the 32 scales.  Tokens >= T
// are written as zero rows (scale 0, codes 0).
__global__ void prefill_fp8_kernel(KvGeom g, uint8_t* kp, uint8_t* vp, const int32_t* pt, const int32_t* lens,
                                   const uint16_t* ks, const uint16_t* vs, int64_t t_stride) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sk = reinterpret_cast<uint16_t*>(smem);
  uint16_t* sv = sk + kSub * g.d;
  float* ssc = reinterpret_cast<float*>(sv + kSub * g.d);  // [2][16]: K scales, V scales
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
    const bool ok = t0 + i / g.d < T;
    sk[i] = ok ? ks[src + i] : (uint16_t)0;
    sv[i] = ok ? vs[src + i] : (uint16_t)0;
  }
  __syncthreads();
  {
    // thread x: row x / 8 of the 32 (K rows 0-15, V rows 16-31), part x % 8
    const int row = threadIdx.x >> 3, part = threadIdx.x & 7;
    const uint16_t* r = (row < kSub ? sk + row * g.d : sv + (row - kSub) * g.d);
    float m = 0.f;
    for (int d = part; d < g.d; d += 8) m = fmaxf(m, fabsf(bf16_to_f32(r[d])));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    if (part == 0) ssc[row] = e4m3_row_scale(m);
  }
  __syncthreads();
  const int nchunk = n / 16;
  for (int c = threadIdx.x; c < nchunk; c += blockDim.x) {
    // K chunk c: token c % 16, head-dim elements 16 (c / 16) .. +16
    const int kt = c % kSub, kd = (c / kSub) * 16;
    const float ksc = ssc[kt];
    u32x4 kw, vw;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const uint16_t* r = sk + kt * g.d + kd + 4 * x;
      kw[x] = e4m3_encode2(bf16_to_f32(r[0]), bf16_to_f32(r[1]), ksc) |
              (e4m3_encode2(bf16_to_f32(r[2]), bf16_to_f32(r[3]), ksc) << 16);
    }
    // V chunk c = (p*4 + j)*16 + i: byte [h*4 + e] = V[4j + e][16(4p + h) + i]
    const int vi = c % 16, vj = (c / 16) % 4, vq = c / 64;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int d = 16 * (4 * vq + h) + vi;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = bf16_to_f32(sv[(4 * vj + e) * g.d + d]);
      // the 4 codes of a word belong to 4 tokens, each with its own scale
      vw[h] = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) vw[h] |= (e4m3_encode2(x[e], 0.f, ssc[kSub + 4 * vj + e]) & 0xFFu) << (8 * e);
    }
    *reinterpret_cast<u32x4*>(kp + base + (int64_t)c * 16) = kw;
    *reinterpret_cast<u32x4*>(vp + base + (int64_t)c * 16) = vw;
  }
  if (threadIdx.x < 2 * kSub) {
    const int64_t si = (phys * g.hkv + gh) * g.page + t0 % g.page + (threadIdx.x % kSub);
    float* dst = scale_ptr(threadIdx.x < kSub ? kp : vp, g);
    dst[si] = ssc[threadIdx.x];
  }
}

__global__ void write_rows_fp8_kernel(KvGeom g, uint8_t* kp, uint8_t* vp, const int32_t* pt, const int32_t* lens,
                                      int batch, const int32_t* rows, const uint16_t* kr, const uint16_t* vr) {
  const int r = blockIdx.x;
  const int b = rows[3 * r], gh = rows[3 * r + 1], t = rows[3 * r + 2];
  if (b < 0 || b >= batch || gh < 0 || gh >= g.hkv || t < 0 || t >= lens[b]) return;
  const int lp = t / g.page;
  if (lp >= g.max_pages) return;
  const int64_t phys = pt[(int64_t)b * g.max_pages + lp];
  const int64_t base = subtile_base(phys, gh, t % g.page, g.hkv, g.page, g.d);
  encode_row_fp8(g, kp, vp, base, t % kSub, (phys * g.hkv + gh) * g.page + t % g.page, kr + (int64_t)r * g.d,
                 vr ? vr + (int64_t)r * g.d : nullptr, threadIdx.x);
}

__global__ void gather_scales_kernel(KvGeom g, const uint8_t* kp, const uint8_t* vp, const int32_t* pt, int b,
                                     int gh, int t0, int n, float* ko, float* vo) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int t = t0 + i;
  const int64_t phys = pt[(int64_t)b * g.max_pages + t / g.page];
  const int64_t si = (phys * g.hkv + gh) * g.page + t % g.page;
  if (ko) ko[i] = reinterpret_cast<const float*>(kp + g.scale_off)[si];
  if (vo) vo[i] = reinterpret_cast<const float*>(vp + g.scale_off)[si];
}

hipError_t launch_append(const KvGeom& g, void* kp, void* vp, const int32_t* pt,
                         const int32_t* lens, const void* kn, const void* vn, int batch,
                         hipStream_t st) {
  if (batch == 0) return hipSuccess;
  dim3 grid(g.hkv, batch);
  if (g.esz == 1)
    hipLaunchKernelGGL(append_fp8_kernel, grid, dim3(64), 0, st, g, (uint8_t*)kp, (uint8_t*)vp, pt, lens,
                       (const uint16_t*)kn, (const uint16_t*)vn);
  else if (g.esz == 2)
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
  if (g.esz == 1) {
    const size_t lds = 2 * (size_t)kSub * g.d * 2 + 2 * kSub * sizeof(float);
    hipLaunchKernelGGL(prefill_fp8_kernel, grid, dim3(256), lds, st, g, (uint8_t*)kp, (uint8_t*)vp, pt, lens,
                       (const uint16_t*)k, (const uint16_t*)v, t_stride);
    return hipGetLastError();
  }
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
  if (g.esz == 1)
    hipLaunchKernelGGL(write_rows_fp8_kernel, dim3(n), dim3(64), 0, st, g, (uint8_t*)kp, (uint8_t*)vp, pt, lens,
                       batch, rows, (const uint16_t*)kr, (const uint16_t*)vr);
  else if (g.esz == 2)
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
  if (g.esz == 1)
    hipLaunchKernelGGL(gather_kernel<uint8_t>, dim3(n), dim3(64), 0, st, g, (const uint8_t*)kp,
                       (const uint8_t*)vp, pt, b, gh, t0, n, (uint8_t*)ko, (uint8_t*)vo);
  else if (g.esz == 2)
    hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(n), dim3(64), 0, st, g, (const uint16_t*)kp,
                       (const uint16_t*)vp, pt, b, gh, t0, n, (uint16_t*)ko, (uint16_t*)vo);
  else
    hipLaunchKernelGGL(gather_kernel<uint32_t>, dim3(n), dim3(64), 0, st, g, (const uint32_t*)kp,
                       (const uint32_t*)vp, pt, b, gh, t0, n, (uint32_t*)ko, (uint32_t*)vo);
  return hipGetLastError();
}

hipError_t launch_gather_scales(const KvGeom& g, const void* kp, const void* vp, const int32_t* pt, int b,
                                int gh, int t0, int n, float* ko, float* vo, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_scales_kernel, dim3((n + 255) / 256), dim3(256), 0, st, g, (const uint8_t*)kp,
                     (const uint8_t*)vp, pt, b, gh, t0, n, ko, vo);
  return hipGetLastError();
}

}  // namespace lak
