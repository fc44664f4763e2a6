// Device fill kernels of the synthetic decode inputs: the same counter-based
// generator as workload/philox.py (Philox4x32-10 of Salmon et al., SC'11, and a
// float64 Box-Muller transform), so that host and device produce identical
// element values.  Built with -ffp-contract=off: every product and sum is rounded
// separately, as in the NumPy code.  No attention arithmetic here.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace {

__device__ inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
    if (r != 9) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
  }
}

// Four normals of block j = e/4 of stream (kind, layer, row).
__device__ inline void normals4(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t row, uint32_t j,
                                double z[4]) {
  uint32_t c[4] = {j, row, layer, kind};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const double u1 = ((double)c[2 * pr] + 1.0) * 2.3283064365386963e-10;
    const double u2 = (double)c[2 * pr + 1] * 2.3283064365386963e-10;
    const double rad = sqrt(-2.0 * log(u1));
    const double th = 6.283185307179586 * u2;
    z[2 * pr] = rad * cos(th);
    z[2 * pr + 1] = rad * sin(th);
  }
}

__device__ inline double normal_at(uint64_t seed, uint32_t kind, uint32_t layer, uint32_t row, uint64_t e) {
  double z[4];
  normals4(seed, kind, layer, row, (uint32_t)(e >> 2), z);
  return z[e & 3];
}

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ inline void store(void* out, int dtype, int64_t i, float v) {
  if (dtype == 0)
    reinterpret_cast<uint16_t*>(out)[i] = bf16_rne(v);
  else
    reinterpret_cast<float*>(out)[i] = v;
}

struct FillArgs {
  void* out;
  int dtype;  // 0 bf16, 1 f32
  int64_t R, T;
  int D;
  const int32_t* t0_rows;  // per-row first position (nullable)
  int64_t t0_const;
  uint32_t kind, layer;
  uint64_t seed;
  int64_t stride_r, stride_t;
  int mode;        // 0 raw, 1 scaled by c1, 2 query: f32(c1 * dir) + f32(c2 * z)
  float c1, c2;
  const float* dirs;  // [R / G][D] for mode 2
  int G;
};

// out[r*stride_r + t*stride_t + d] for r < R, t < T, d < D; 4 elements per thread.
__global__ void fill_tokens_kernel(FillArgs a) {
  const int64_t quads = a.R * a.T * (a.D / 4);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < quads;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int dq = (int)(i % (a.D / 4));
    const int64_t rt = i / (a.D / 4);
    const int64_t t = rt % a.T;
    const int64_t r = rt / a.T;
    const int64_t t0 = a.t0_rows ? a.t0_rows[r] : a.t0_const;
    const uint64_t e = (uint64_t)(t0 + t) * a.D + 4 * dq;
    double z[4];
    normals4(a.seed, a.kind, a.layer, (uint32_t)r, (uint32_t)(e >> 2), z);
    const int64_t base = r * a.stride_r + t * a.stride_t + 4 * dq;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float z32 = __double2float_rn(z[x]);
      float v = z32;
      if (a.mode == 1) v = __fmul_rn(z32, a.c1);
      if (a.mode == 2)
        v = __fadd_rn(__fmul_rn(a.c1, a.dirs[(r / a.G) * a.D + 4 * dq + x]), __fmul_rn(a.c2, z32));
      store(a.out, a.dtype, base + x, v);
    }
  }
}

struct SalientArgs {
  void* out;
  int dtype;
  int64_t R;
  int npos, D;
  const int32_t* pos;  // [R][npos]
  const float* dirs;   // [R][D]
  int64_t t_begin, t_count;
  int64_t stride_r, stride_t;
  uint32_t kind, layer;
  uint64_t seed;
  float strength;
};

// Salient keys: out = f32(strength * dir) + f32(noise) at the listed positions.
__global__ void apply_salient_kernel(SalientArgs a) {
  const int64_t ri = blockIdx.x;  // r * npos + i
  const int64_t r = ri / a.npos;
  const int64_t p = a.pos[ri];
  if (p < a.t_begin || p >= a.t_begin + a.t_count) return;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    const float z32 = __double2float_rn(normal_at(a.seed, a.kind, a.layer, (uint32_t)r, (uint64_t)p * a.D + d));
    const float v = __fadd_rn(__fmul_rn(a.strength, a.dirs[r * a.D + d]), z32);
    store(a.out, a.dtype, r * a.stride_r + (p - a.t_begin) * a.stride_t + d, v);
  }
}

struct RowsArgs {
  void* out;  // [n][D]
  int dtype;
  int n, D;
  const int32_t* rows;  // stream row of each output row
  const int32_t* toks;  // position of each output row
  const float* dirs;    // [n][D] salient direction or NULL; row i salient iff salient[i]
  const int32_t* salient;
  uint32_t kind, layer;
  uint64_t seed;
  float strength;
};

__global__ void fill_rows_kernel(RowsArgs a) {
  const int i = blockIdx.x;
  if (i >= a.n) return;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    const float z32 = __double2float_rn(
        normal_at(a.seed, a.kind, a.layer, (uint32_t)a.rows[i], (uint64_t)a.toks[i] * a.D + d));
    float v = z32;
    if (a.dirs && a.salient && a.salient[i]) v = __fadd_rn(__fmul_rn(a.strength, a.dirs[(int64_t)i * a.D + d]), z32);
    store(a.out, a.dtype, (int64_t)i * a.D + d, v);
  }
}

}  // namespace

extern "C" {

// Returns 0 on success, a hipError_t value otherwise.
int wl_fill_tokens(void* out, int dtype, int64_t R, int64_t T, int D, const int32_t* t0_rows, int64_t t0_const,
                   int kind, int layer, uint64_t seed, int64_t stride_r, int64_t stride_t, int mode, float c1,
                   float c2, const float* dirs, int G, void* stream) {
  if (R <= 0 || T <= 0) return 0;
  if (D % 4 != 0 || !out) return (int)hipErrorInvalidValue;
  FillArgs a{out, dtype, R, T, D, t0_rows, t0_const, (uint32_t)kind, (uint32_t)layer, seed, stride_r, stride_t,
             mode, c1, c2, dirs, G > 0 ? G : 1};
  const int64_t quads = R * T * (D / 4);
  const int64_t blocks = std::min<int64_t>((quads + 255) / 256, 1 << 20);
  hipLaunchKernelGGL(fill_tokens_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int wl_apply_salient(void* out, int dtype, int64_t R, int npos, int D, const int32_t* pos, const float* dirs,
                     int64_t t_begin, int64_t t_count, int64_t stride_r, int64_t stride_t, int kind, int layer,
                     uint64_t seed, float strength, void* stream) {
  if (R <= 0 || npos <= 0) return 0;
  SalientArgs a{out, dtype, R, npos, D, pos, dirs, t_begin, t_count, stride_r, stride_t, (uint32_t)kind,
                (uint32_t)layer, seed, strength};
  hipLaunchKernelGGL(apply_salient_kernel, dim3((unsigned)(R * npos)), dim3(128), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int wl_fill_rows(void* out, int dtype, int n, int D, const int32_t* rows, const int32_t* toks, const float* dirs,
                 const int32_t* salient, int kind, int layer, uint64_t seed, float strength, void* stream) {
  if (n <= 0) return 0;
  RowsArgs a{out, dtype, n, D, rows, toks, dirs, salient, (uint32_t)kind, (uint32_t)layer, seed, strength};
  hipLaunchKernelGGL(fill_rows_kernel, dim3(n), dim3(128), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // extern "C"
