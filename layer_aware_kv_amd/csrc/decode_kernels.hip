// Split-K decode attention over the paged KV cache, for the three layer tiers of
// DELTA ("Methodology in Plain English", DELTA AI summary page):
//   MODE_FULL   full attention (layers 0-1),
//   MODE_DELTA  full attention that also writes what the page scores need of every
//               valid token's logit (the delta-layer scores are taken from the decode
//               kernel's own logits, as the pages' implementation does): per head and
//               16-token sub-tile the max logit and fp16 weights relative to it (MAX
//               aggregation), or the (max, sum of exponentials) pair (SUM),
//   MODE_SPARSE attention over the tokens of the selected pages only.
// One workgroup = one (sequence b, KV head g, split s); a row's pages are dealt to
// its splits round-robin and a split's 4 waves take its pages in turn.  Per
// sub-tile: S^T = K Q^T with the G query heads of the group as the 16-wide MFMA N
// dimension, online softmax in the log2 domain, then O^T += V^T P^T.  K and V
// fragments come straight from HBM into registers (the pool's in-page order matches
// the MFMA operand layout, so every load instruction is one contiguous 1 KiB); fp8
// pools are widened to bfloat16 in registers.  Waves merge through LDS; the split
// partials (o, max, sum) are merged by combine_kernel.
#include <math.h>

#include <algorithm>

#include <hip/hip_ext.h>

#include "lak_combine.h"
#include "lak_device.h"
#include "lak_internal.h"

namespace lak {

// 16-byte fragment load, non-temporal: K/V pages are read once per call, so they do
// not evict from the caches what is reused soon (the delta-layer scratch, the page
// table, the selection, the partials).
__device__ inline u32x4 load16(const u32x4* p) { return __builtin_nontemporal_load(p); }

template <int ESZ, int D>
struct Frag;

// bfloat16: q.K^T with v_mfma_f32_16x16x32_bf16 (D/32 per sub-tile), P.V with
// v_mfma_f32_16x16x16_bf16 (D/16 per sub-tile).
template <int D>
struct Frag<2, D> {
  static constexpr int NL = D / 32;  // 16-byte loads per lane per operand
  static constexpr int NO = D / 16;  // 16-row output tiles of O^T
  static constexpr int NQ = D / 32;  // q operands
  u32x4 k[NL], v[NL];
  typedef bf16x8 QF;

  __device__ inline void load(const uint16_t* kb, const uint16_t* vb, const float*, const float*, int lane) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(kb);
    const u32x4* vp = reinterpret_cast<const u32x4*>(vb);
#pragma unroll
    for (int i = 0; i < NL; ++i) k[i] = load16(kp + i * 64 + lane);
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = load16(vp + i * 64 + lane);
  }
  // lane l: head l%16, head-dim chunk (4i + l/16)*8 .. +8
  __device__ static inline void load_q(QF* qf, const uint16_t* qrow, bool valid, int j) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid) w = *reinterpret_cast<const u32x4*>(qrow + 32 * i + 8 * j);
      qf[i] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __device__ inline f32x4 qk(const QF* qf) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k[i]), qf[i], s, 0, 0, 0);
    return s;
  }
  // zero the V elements of tokens >= nvalid (token of element x is 4(l/16) + x%4)
  __device__ inline void mask_v(int nvalid, int j) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (4 * j + e >= nvalid) {
        const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          v[i][e >> 1] &= keep;
          v[i][2 + (e >> 1)] &= keep;
        }
      }
    }
  }
  // replace token tt of this sub-tile by the row (kr, vr) in the fragments
  __device__ inline void patch(const uint16_t* kr, const uint16_t* vr, int tt, int lane) {
    const int n = lane & 15, j = lane >> 4;
    if (n == tt) {
#pragma unroll
      for (int i = 0; i < NL; ++i) k[i] = *reinterpret_cast<const u32x4*>(kr + (4 * i + j) * 8);
    }
    if (j == tt / 4) {
      uint32_t val[NL][2];  // every load issued before the first is used
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) val[i][h] = vr[16 * (2 * i + h) + n];
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)  // compile-time element index
            if (e == (tt & 3)) {
              const int x = h * 4 + e, sh = 16 * (x & 1);
              v[i][x >> 1] = (v[i][x >> 1] & ~(0xFFFFu << sh)) | (val[i][h] << sh);
            }
    }
  }
  __device__ inline void pv(f32x4* o, const float* p) const {
    const uint32_t w0 = (uint32_t)f32_to_bf16_rne(p[0]) | ((uint32_t)f32_to_bf16_rne(p[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16_rne(p[2]) | ((uint32_t)f32_to_bf16_rne(p[3]) << 16);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const i16x4 pf = __builtin_bit_cast(i16x4, (u32x2){w0, w1});
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const i16x4 va = __builtin_bit_cast(i16x4, (u32x2){v[i][0], v[i][1]});
      const i16x4 vb = __builtin_bit_cast(i16x4, (u32x2){v[i][2], v[i][3]});
      o[2 * i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pf, o[2 * i], 0, 0, 0);
      o[2 * i + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb, pf, o[2 * i + 1], 0, 0, 0);
    }
  }
};

// float32: v_mfma_f32_16x16x4_f32 for both products (D/4 each per sub-tile).
template <int D>
struct Frag<4, D> {
  static constexpr int NL = D / 16;
  static constexpr int NO = D / 16;
  static constexpr int NQ = D / 16;
  u32x4 k[NL], v[NL];
  typedef f32x4 QF;

  __device__ inline void load(const uint32_t* kb, const uint32_t* vb, const float*, const float*, int lane) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(kb);
    const u32x4* vp = reinterpret_cast<const u32x4*>(vb);
#pragma unroll
    for (int i = 0; i < NL; ++i) k[i] = load16(kp + i * 64 + lane);
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = load16(vp + i * 64 + lane);
  }
  // lane l: head l%16, head-dim elements 16i + 4(l/16) .. +4
  __device__ static inline void load_q(QF* qf, const uint32_t* qrow, bool valid, int j) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
      if (valid) w = *reinterpret_cast<const f32x4*>(qrow + 16 * i + 4 * j);
      qf[i] = w;
    }
  }
  __device__ inline f32x4 qk(const QF* qf) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(k[i][e]), qf[i][e], s, 0, 0, 0);
    return s;
  }
  __device__ inline void mask_v(int nvalid, int j) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * j + e >= nvalid) {
#pragma unroll
        for (int i = 0; i < NL; ++i) v[i][e] = 0u;
      }
  }
  __device__ inline void patch(const uint32_t* kr, const uint32_t* vr, int tt, int lane) {
    const int n = lane & 15, j = lane >> 4;
    if (n == tt) {
#pragma unroll
      for (int i = 0; i < NL; ++i) k[i] = *reinterpret_cast<const u32x4*>(kr + (4 * i + j) * 4);
    }
    if (j == tt / 4) {
      uint32_t val[NL];  // every load issued before the first is used
#pragma unroll
      for (int i = 0; i < NL; ++i) val[i] = vr[16 * i + n];
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)  // compile-time element index (a runtime one goes to scratch)
          if (e == (tt & 3)) v[i][e] = val[i];
    }
  }
  __device__ inline void pv(f32x4* o, const float* p) const {
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v[i][e]), p[e], o[i], 0, 0, 0);
  }
};

// fp8 (OCP E4M3 codes, one float32 scale per token): the codes are widened to
// bfloat16 in registers (exact: every E4M3 value is a bfloat16 value) and go
// through the same bf16 MFMAs; the key scale of a token multiplies its logit and
// the value scale its probability, so no element is rescaled.
template <int D>
struct Frag<1, D> {
  static constexpr int NL = D / 64;  // 16-byte loads per lane per operand
  static constexpr int NO = D / 16;
  static constexpr int NQ = D / 32;
  u32x4 k[NL], v[NL];
  u32x4 ks, vs;  // float bits of the key / value scales of tokens 4(l/16) .. +4
  typedef bf16x8 QF;

  __device__ inline void load(const uint8_t* kb, const uint8_t* vb, const float* ksb, const float* vsb,
                              int lane) {
    const u32x4* kp = reinterpret_cast<const u32x4*>(kb);
    const u32x4* vp = reinterpret_cast<const u32x4*>(vb);
#pragma unroll
    for (int i = 0; i < NL; ++i) k[i] = load16(kp + i * 64 + lane);
#pragma unroll
    for (int i = 0; i < NL; ++i) v[i] = load16(vp + i * 64 + lane);
    ks = load16(reinterpret_cast<const u32x4*>(ksb) + (lane >> 4));
    vs = load16(reinterpret_cast<const u32x4*>(vsb) + (lane >> 4));
  }
  // Lane l of load i holds token l%16, head-dim elements 16(4i + l/16) .. +16; the
  // first 8 feed MFMA 2i, the other 8 MFMA 2i+1, so q operand m of lane l holds
  // head l%16, elements 64(m/2) + 16(l/16) + 8(m%2) .. +8.
  __device__ static inline void load_q(QF* qf, const uint16_t* qrow, bool valid, int j) {
#pragma unroll
    for (int m = 0; m < NQ; ++m) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (valid) w = *reinterpret_cast<const u32x4*>(qrow + 64 * (m >> 1) + 16 * j + 8 * (m & 1));
      qf[m] = __builtin_bit_cast(bf16x8, w);
    }
  }
  // 2 E4M3 codes (bytes 0-1, or 2-3 for HI) of a word -> 2 bfloat16 in one word
  template <bool HI>
  __device__ static inline uint32_t widen2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  __device__ inline f32x4 qk(const QF* qf) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 a = {widen2<false>(k[i][2 * h]), widen2<true>(k[i][2 * h]), widen2<false>(k[i][2 * h + 1]),
                         widen2<true>(k[i][2 * h + 1])};
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), qf[2 * i + h], s, 0, 0, 0);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] *= __uint_as_float(ks[r]);
    return s;
  }
  // zero the codes of tokens >= nvalid (token of byte e of a word is 4(l/16) + e)
  __device__ inline void mask_v(int nvalid, int j) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * j + e >= nvalid) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int x = 0; x < 4; ++x) v[i][x] &= ~(0xFFu << (8 * e));
      }
  }
  // Word x of load i holds the codes of tokens 4(l/16) .. +4 at head-dim element
  // 16(4i + x) + l%16: the A operand of output tile 4i + x.
  __device__ inline void pv(f32x4* o, const float* p) const {
    float w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = (p[r] == 0.f) ? 0.f : p[r] * __uint_as_float(vs[r]);
    const uint32_t w0 = (uint32_t)f32_to_bf16_rne(w[0]) | ((uint32_t)f32_to_bf16_rne(w[1]) << 16);
    const uint32_t w1 = (uint32_t)f32_to_bf16_rne(w[2]) | ((uint32_t)f32_to_bf16_rne(w[3]) << 16);
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const i16x4 pf = __builtin_bit_cast(i16x4, (u32x2){w0, w1});
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const i16x4 va = __builtin_bit_cast(i16x4, (u32x2){widen2<false>(v[i][x]), widen2<true>(v[i][x])});
        o[4 * i + x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pf, o[4 * i + x], 0, 0, 0);
      }
  }
};

template <int ESZ>
struct ElemT;
template <>
struct ElemT<1> { typedef uint8_t T; };
template <>
struct ElemT<2> { typedef uint16_t T; };
template <>
struct ElemT<4> { typedef uint32_t T; };

// At least 4 waves per SIMD for the single-sub-tile batch (register budget 128); fp32
// fragments (q, K, V and the output accumulator at 32 registers each for D = 128) take the
// 3-wave budget instead of spilling.
template <int ESZ, int D, int MODE, int U>
__global__ __launch_bounds__(256, (U == 1 && ESZ != 4 ? 4 : (U <= 2 ? 3 : 2))) void decode_kernel(DecodeArgs a) {
  typedef typename ElemT<ESZ>::T E;
  typedef typename ElemT<ESZ == 1 ? 2 : ESZ>::T QE;  // q rows: bfloat16 for fp8 pools
  typedef Frag<ESZ, D> F;
  extern __shared__ __align__(16) float lds[];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.hq / a.hkv;
  const int Gp = G + (G & 1);
  const int T = a.seq_lens[b];
  const int P = a.page;
  const int NP = (T + P - 1) / P;

  int n_items = NP;
  const int32_t* sel_row = nullptr;
  if (MODE == MODE_SPARSE) {
    const int64_t row = (int64_t)b * a.sel_rows + (a.sel_rows == 1 ? 0 : g);
    n_items = min(max(a.sel_count[row], 0), min(a.sel_cap, NP));
    sel_row = a.sel + row * a.sel_cap;
  }
  // Fused append.  The wave whose items include the page of this step's token (T-1)
  // stores that row into the pool itself before its loads (below) -- or, on the delta
  // tier of bfloat16 / fp32 pools, patches it into its fragments (`patch`).  On the full
  // tier (and the fp8 delta tier) that wave always exists, since every page is an item,
  // and its store is the append.  Where it may not store (delta patch; a sparse
  // selection without the token's page), split 0 of the row also writes the row, at the
  // end of the kernel: nothing in this call reads it from the pool but that wave, so the
  // store does not delay the split's own loads.  Both write the same bytes.
  // (fp8 pools: rows arrive as bfloat16 and are encoded with their row scale.)
  const QE* krow_new = nullptr;
  const QE* vrow_new = nullptr;
  if (a.k_new != nullptr && T > 0) {
    krow_new = reinterpret_cast<const QE*>(a.k_new) + ((int64_t)b * a.hkv + g) * D;
    vrow_new = reinterpret_cast<const QE*>(a.v_new) + ((int64_t)b * a.hkv + g) * D;
  }
  constexpr bool kOwnerStores = (ESZ == 1 || MODE != MODE_DELTA);
  const bool split0_store = krow_new != nullptr && s == 0 && (MODE == MODE_SPARSE || !kOwnerStores);
  auto store_token = [&]() {
    const int t = T - 1;
    const int64_t phys = a.page_table[(int64_t)b * a.max_pages + t / P];
    const int64_t row0 = (phys * a.hkv + g) * P + ((t % P) / kSub) * kSub;  // sub-tile's first row
    E* kp = const_cast<E*>(reinterpret_cast<const E*>(a.k_pool));
    E* vp = const_cast<E*>(reinterpret_cast<const E*>(a.v_pool));
    if constexpr (ESZ == 1) {
      if (threadIdx.x < 64)
        encode_rows_fp8(D, kp + row0 * D, vp + row0 * D, t % kSub, const_cast<float*>(a.k_scale) + row0 + t % kSub,
                        const_cast<float*>(a.v_scale) + row0 + t % kSub, krow_new, vrow_new, threadIdx.x);
    } else {
      for (int d = threadIdx.x; d < D; d += blockDim.x) {
        kp[row0 * D + k_off<ESZ>(t % kSub, d)] = krow_new[d];
        vp[row0 * D + v_off<ESZ>(t % kSub, d)] = vrow_new[d];
      }
    }
  };

  // The row's items are dealt round-robin to its S_row splits (split s takes items
  // s, s + S_row, s + 2 S_row, ...): the workgroups of a row then stream neighbouring
  // pages at the same time, which keeps concurrent DRAM accesses close together.
  const int S_row = (n_items + a.pps - 1) / a.pps;
  if (s >= S_row) {
    if (split0_store) store_token();  // a row with no items (empty selection)
    return;
  }
  const int n_split = (n_items - s + S_row - 1) / S_row;  // items of this split

  // wave index made wave-uniform so that all per-sub-tile bookkeeping is scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, j = lane >> 4;
  const bool head_ok = n < G;

  typename F::QF qf[F::NQ];
  F::load_q(qf, reinterpret_cast<const QE*>(a.q) + ((int64_t)b * a.hq + g * G + (head_ok ? n : 0)) * D,
            head_ok, j);

  const E* kpool = reinterpret_cast<const E*>(a.k_pool);
  const E* vpool = reinterpret_cast<const E*>(a.v_pool);
  const int32_t* ptab = a.page_table + (int64_t)b * a.max_pages;
  const int spp = P / kSub;
  const float qk_scale2 = a.sm_scale * kLog2e;

  // This wave takes members wave + kWaves*k (k < n_w <= 64 * kIdRegs: the host caps
  // the items per split at 256, 512 for the full tier) of its split.  Lane k % 64
  // fetches the logical and physical page of item k once into register k / 64; each
  // sub-tile then reads them with v_readlane (no memory access in the loop).
  constexpr int kIdRegs = (MODE == MODE_FULL) ? 2 : 1;
  const int n_w = max(0, (n_split - wave + kWaves - 1) / kWaves);
  const int nsub = n_w * spp;
  int lp_vec[kIdRegs], pid_vec[kIdRegs];
#pragma unroll
  for (int r = 0; r < kIdRegs; ++r) {
    lp_vec[r] = -1;
    pid_vec[r] = 0;
    if (lane + 64 * r < n_w) {
      const int it = s + S_row * (wave + kWaves * (lane + 64 * r));
      int lp = (MODE == MODE_SPARSE) ? sel_row[it] : it;
      if (lp >= 0 && lp < NP) {
        lp_vec[r] = lp;
        pid_vec[r] = ptab[lp];
      }
    }
  }
  auto item_lp = [&](int k) -> int {
    return (kIdRegs == 1 || k < 64) ? __builtin_amdgcn_readlane(lp_vec[0], k & 63)
                                    : __builtin_amdgcn_readlane(lp_vec[kIdRegs - 1], k & 63);
  };
  auto item_pid = [&](int k) -> int {
    return (kIdRegs == 1 || k < 64) ? __builtin_amdgcn_readlane(pid_vec[0], k & 63)
                                    : __builtin_amdgcn_readlane(pid_vec[kIdRegs - 1], k & 63);
  };

  // The ids (and q) are in registers before the loop: wait for them once here, so
  // that reading them inside the loop never waits on the K/V loads in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // The wave whose items include the page of this step's token stores that row itself
  // (fp8 pools: encoded) before any of its loads, so it then reads the token from the
  // pool like any other; a workgroup-scope fence, just before it loads the token's
  // sub-tile (x_tok), orders its lanes' stores before that load.  This keeps the
  // sub-tile loop free of the register patch, whose extra loads force conservative
  // wait counts on every sub-tile (full tier 332 -> 324 us at B 16, T 64k); the delta
  // tier of bfloat16 / fp32 pools keeps the patch, which measured faster there.
  int x_tok = -1;
  if constexpr (kOwnerStores) {
    if (krow_new != nullptr) {
      unsigned long long own = 0ull;
      int k_own = 0;
#pragma unroll
      for (int r = kIdRegs - 1; r >= 0; --r) {
        const unsigned long long o = __ballot(lp_vec[r] == (T - 1) / P);
        if (o != 0ull) {
          own = o;
          k_own = 64 * r + __ffsll(o) - 1;
        }
      }
      if (own != 0ull) {
        const int64_t phys = item_pid(k_own);
        const int tin = (T - 1) % P;
        const int64_t row0 = (phys * a.hkv + g) * P + (tin / kSub) * kSub;
        const int tt = tin % kSub;
        if constexpr (ESZ == 1) {
          encode_rows_fp8(D, const_cast<E*>(kpool) + row0 * D, const_cast<E*>(vpool) + row0 * D, tt,
                          const_cast<float*>(a.k_scale) + row0 + tt, const_cast<float*>(a.v_scale) + row0 + tt,
                          krow_new, vrow_new, lane);
        } else {
          for (int d = lane; d < D; d += 64) {
            const_cast<E*>(kpool)[row0 * D + k_off<ESZ>(tt, d)] = krow_new[d];
            const_cast<E*>(vpool)[row0 * D + v_off<ESZ>(tt, d)] = vrow_new[d];
          }
        }
        x_tok = k_own * spp + tin / kSub;
      }
    }
  }

  struct Sub {
    bool valid;
    int t0;
  };
  // Issues the K/V loads of sub-tile x (< nsub).  The loads are issued even for a
  // sub-tile that has no valid token (then from the pool's first sub-tile, always
  // mapped) so that the steady-state loop issues the same loads on every path.
  auto issue = [&](F& f, int x) -> Sub {
    const int k = x / spp;
    const int sub = x - k * spp;
    const int lp = item_lp(k);
    const int t0 = lp * P + sub * kSub;
    const bool valid = lp >= 0 && t0 < T;
    const int64_t phys = item_pid(k);
    const int64_t row0 = valid ? (phys * a.hkv + g) * P + sub * kSub : 0;  // first token row
    f.load(kpool + row0 * D, vpool + row0 * D, a.k_scale + row0, a.v_scale + row0, lane);
    return Sub{valid, t0};
  };

  // delta tier, MAX: bytes of one sub-tile's block (weights [G][16] fp16, then G maxima)
  const int blk_bytes = max_block_bytes(G);

  float m2 = -INFINITY;  // running max, log2 units
  float l = 0.f;         // this lane's share of the running sum
  f32x4 o[F::NO];
#pragma unroll
  for (int x = 0; x < F::NO; ++x) o[x] = (f32x4){0.f, 0.f, 0.f, 0.f};

  auto process = [&](F& f, int ct, int x) {
    if constexpr (ESZ != 1 && MODE == MODE_DELTA) {
      if (krow_new != nullptr && T - 1 < ct + kSub) f.patch(krow_new, vrow_new, (T - 1) - ct, lane);
    }
    const f32x4 sacc = f.qk(qf);
    const int tb = ct + 4 * j;
    float s2[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s2[r] = (tb + r < T) ? sacc[r] * qk_scale2 : -INFINITY;
      mx = fmaxf(mx, s2[r]);
    }
    mx = xor32_max(xor16_max(mx));
    const float m_new = fmaxf(m2, mx);
    const float alpha = exp2f(m2 - m_new);
    float p[4];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = exp2f(s2[r] - m_new);
      ps += p[r];
    }
    // delta tier: weights relative to this sub-tile's max, 2^(logit - mx) = p * 2^(m_new - mx);
    // taken from p unless the running max is so far above mx (> 2^64) that p could lose
    // precision, then computed directly
    const float to_rel = exp2f(m_new - mx);
    const bool rel_from_p = (m_new - mx) <= 64.f;
    if (MODE == MODE_DELTA && a.sum_pairs) {
      // (r, e) of this head over the sub-tile: r = max logit (log2 units), e = sum of
      // 2^(logit - r); the page score later is sum_h e * exp(r ln 2 - lse_h)
      float e = 0.f;
      if (rel_from_p) {
        e = ps * to_rel;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) e += exp2f(s2[r] - mx);
      }
      e = xor32_add(xor16_add(e));
      if (head_ok && j == 0) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        if (a.lds_stage) {
          // staged at the sub-tile's index within the workgroup; flushed at the end
          const int li = (wave + kWaves * (x / spp)) * spp + (x % spp);
          *reinterpret_cast<f32x2*>(lds + (li * Gp + n) * 2) = (f32x2){mx, e};
        } else {
          const int64_t blk = ((int64_t)b * a.hkv + g) * (a.t_pad / kSub) + ct / kSub;
          *reinterpret_cast<f32x2*>(a.pairs + (blk * Gp + n) * 2) = (f32x2){mx, e};
        }
      }
    } else if (MODE == MODE_DELTA && head_ok) {
      // MAX aggregation: this head's max logit r over the sub-tile (log2 units, exact)
      // and each token's weight relative to it, u = 2^(logit - r) in (0, 1], rounded to
      // fp16; the page score later is sum_t max_h u * 2^(r - lse_h), so its relative
      // error is at most 2^-11.  One block per sub-tile: [G heads][16 tokens] weights,
      // then the G maxima (only the group's real heads: no padding head is written).
      uint32_t hw[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float u0 = rel_from_p ? p[2 * r] * to_rel : exp2f(s2[2 * r] - mx);
        const float u1 = rel_from_p ? p[2 * r + 1] * to_rel : exp2f(s2[2 * r + 1] - mx);
        hw[r] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)u0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)u1) << 16);
      }
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      uint8_t* dst;
      if (a.lds_stage) {
        // staged in LDS at the sub-tile's index within the workgroup; flushed at the end
        const int li = (wave + kWaves * (x / spp)) * spp + (x % spp);
        dst = reinterpret_cast<uint8_t*>(lds) + (size_t)li * blk_bytes;
      } else {
        const int64_t blk = ((int64_t)b * a.hkv + g) * (a.t_pad / kSub) + ct / kSub;
        dst = a.rel_blk + blk * blk_bytes;
      }
      *reinterpret_cast<u32x2*>(dst + n * (kSub * 2) + 8 * j) = (u32x2){hw[0], hw[1]};
      if (j == 0) *reinterpret_cast<float*>(dst + G * (kSub * 2) + 4 * n) = mx;
    }
    l = l * alpha + ps;
    m2 = m_new;
#pragma unroll
    for (int x = 0; x < F::NO; ++x) o[x] *= alpha;
    if (ct + kSub > T) f.mask_v(T - ct, j);
    f.pv(o, p);
  };

  // U sub-tiles per batch: their loads are issued together (unconditionally, so
  // the wait before each sub-tile is exact) and consumed in order; other waves of
  // the CU cover the latency between batches.  (A two-buffer pipeline that keeps
  // the next sub-tile's loads in flight during the math measured slower: it costs
  // occupancy, and occupancy hides the latency better.)
  for (int x = 0; x < nsub; x += U) {
    if (kOwnerStores && x_tok >= x && x_tok < x + U) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
    F buf[U];
    Sub info[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      info[u] = issue(buf[u], min(x + u, nsub - 1));
      info[u].valid = info[u].valid && (x + u < nsub);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (info[u].valid) process(buf[u], info[u].t0, x + u);
  }

  if (MODE == MODE_DELTA && a.lds_stage && !a.sum_pairs) {
    // write the workgroup's blocks in one burst, 16 bytes per thread: each block is
    // contiguous (its tail past the maxima, if any, is padding and never read)
    __syncthreads();
    const int n_sub = n_split * spp;
    const int upb = blk_bytes / 16;  // 16-byte units per block
    for (int idx = threadIdx.x; idx < n_sub * upb; idx += blockDim.x) {
      const int li = idx / upb, u = idx - li * upb;
      const int member = li / spp, sub = li - member * spp;
      const int t0 = (s + S_row * member) * P + sub * kSub;
      if (t0 < T) {
        const int64_t blk = ((int64_t)b * a.hkv + g) * (a.t_pad / kSub) + t0 / kSub;
        *reinterpret_cast<u32x4*>(a.rel_blk + blk * blk_bytes + 16 * u) =
            *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(lds) + (size_t)li * blk_bytes + 16 * u);
      }
    }
    __syncthreads();  // the merge below reuses this LDS
  }
  if (MODE == MODE_DELTA && a.lds_stage && a.sum_pairs) {
    // SUM: the workgroup's (max, sum) pairs, 16-byte units (two heads each); a padding
    // head's pair is never read
    __syncthreads();
    const int n_sub = n_split * spp;
    const int upb = Gp / 2;  // units per sub-tile block
    for (int idx = threadIdx.x; idx < n_sub * upb; idx += blockDim.x) {
      const int li = idx / upb, u = idx - li * upb;
      const int member = li / spp, sub = li - member * spp;
      const int t0 = (s + S_row * member) * P + sub * kSub;
      if (t0 < T) {
        const int64_t blk = ((int64_t)b * a.hkv + g) * (a.t_pad / kSub) + t0 / kSub;
        *reinterpret_cast<u32x4*>(a.pairs + blk * Gp * 2 + 4 * u) =
            *reinterpret_cast<const u32x4*>(lds + li * Gp * 2 + 4 * u);
      }
    }
    __syncthreads();  // the merge below reuses this LDS
  }

  l = xor32_add(xor16_add(l));

  // merge the waves of this workgroup through LDS
  float* lo = lds;                       // [kWaves][G][D]
  float* lm = lds + kWaves * G * D;      // [kWaves][16]
  float* ll = lm + kWaves * 16;          // [kWaves][16]
  if (head_ok) {
#pragma unroll
    for (int x = 0; x < F::NO; ++x)
      *reinterpret_cast<f32x4*>(lo + (wave * G + n) * D + 16 * x + 4 * j) = o[x];
    if (j == 0) {
      lm[wave * 16 + n] = m2;
      ll[wave * 16 + n] = l;
    }
  }
  __syncthreads();
  // 4 consecutive head-dim elements per thread (one pass for G * D <= 1024): the
  // waves' weights are taken once per 4 elements and the partial row is written in
  // 16-byte stores.
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  for (int idx = threadIdx.x; idx < G * D / 4; idx += blockDim.x) {
    const int hn = (4 * idx) / D, d = 4 * idx - hn * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lm[w * 16 + hn]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(lm[w * 16 + hn] - M);
        acc += f * *reinterpret_cast<const f32x4*>(lo + (w * G + hn) * D + d);
        L += f * ll[w * 16 + hn];
      }
    }
    const int64_t row = ((int64_t)b * a.hq + g * G + hn) * a.s_cap + s;
    *reinterpret_cast<f32x4*>(a.o_part + row * D + d) = acc;
    if (d == 0) *reinterpret_cast<f32x2*>(a.ml_part + row * 2) = (f32x2){M, L};
  }
  if (split0_store) store_token();
}

// One wave per (head, sequence); NF: splits loaded in one round (0: the looped path).
template <int ESZ, int D, int NF>
__global__ __launch_bounds__(64) void combine_kernel(CombineArgs a) {
  combine_head<ESZ, D, NF>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// With trace events the kernel is launched with them attached to its own dispatch
// (hipExtLaunchKernelGGL): `ev0` / `ev1` take the kernel's start and end times, so
// their difference is the kernel's execution, with no separate event packets around it.
template <int ESZ, int D, int MODE, int U>
static void launch_decode_m(const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1) {
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((decode_kernel<ESZ, D, MODE, U>), grid, dim3(256), (uint32_t)lds, st, ev0, ev1, 0u, a);
  else
    hipLaunchKernelGGL((decode_kernel<ESZ, D, MODE, U>), grid, dim3(256), lds, st, a);
}

template <int ESZ, int D, int U>
static void launch_decode_u(int mode, const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1) {
  if (mode == MODE_FULL)
    launch_decode_m<ESZ, D, MODE_FULL, U>(a, grid, lds, st, ev0, ev1);
  else if (mode == MODE_DELTA)
    launch_decode_m<ESZ, D, MODE_DELTA, U>(a, grid, lds, st, ev0, ev1);
  else
    launch_decode_m<ESZ, D, MODE_SPARSE, U>(a, grid, lds, st, ev0, ev1);
}

template <int ESZ, int D>
static hipError_t launch_decode_t(int mode, const DecodeArgs& a, int splits, int batch, hipStream_t st,
                                  hipEvent_t ev0, hipEvent_t ev1) {
  const int G = a.hq / a.hkv;
  size_t lds = (size_t)(kWaves * G * D + 2 * kWaves * 16) * sizeof(float);
  if (mode == MODE_DELTA && a.lds_stage)
    lds = std::max(lds, delta_stage_bytes(a.pps, a.page, G, a.sum_pairs != 0));
  dim3 grid(splits, a.hkv, batch);
  // fp32 pools always load one sub-tile at a time: their fragments fill the register
  // budget of a deeper batch.
  int u = ESZ == 4 ? 1 : tune_decode_batch(mode);
  if (u == 0) {
    if (ESZ == 1 && (mode == MODE_SPARSE || (mode == MODE_DELTA && 4 * lds > kLdsBytesPerCu))) {
      // fp8 pools (half the bytes and registers per sub-tile): two sub-tiles per batch on
      // the sparse tier, and on the delta tier where its LDS stage already holds a CU to
      // three workgroups, so the deeper batch's registers cost no occupancy (B 16,
      // 64k-context stack +0.4% and +1.8%; at B 8, 16k context, where the delta stage is
      // small, the delta tier's two per batch cost 5%; the full tier keeps one: two cost
      // it 0.7%)
      u = 2;
    } else if (mode == MODE_SPARSE) {
      // sparse tier, by split size: a wave whose whole share is at most two sub-tiles loads
      // it in one batch (one memory round trip per wave; a B 8, 16k-context stack +1.2%);
      // longer shares keep one sub-tile per batch and the four waves per SIMD that hide
      // their latency better (two per batch: B 16, 64k-context stack -1.3%)
      const int per_wave = (a.pps + kWaves - 1) / kWaves * (a.page / kSub);
      u = per_wave <= 2 ? 2 : 1;
    } else {
      u = 1;  // bfloat16 delta tier: two per batch cost the B 16, 64k-context stack 1.0%
    }
  }
  if constexpr (ESZ != 4) {
    if (u == 4) {
      launch_decode_u<ESZ, D, 4>(mode, a, grid, lds, st, ev0, ev1);
      return hipGetLastError();
    }
    if (u == 2) {
      launch_decode_u<ESZ, D, 2>(mode, a, grid, lds, st, ev0, ev1);
      return hipGetLastError();
    }
  }
  launch_decode_u<ESZ, D, 1>(mode, a, grid, lds, st, ev0, ev1);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, int mode, int D, const DecodeArgs& a, int splits, int batch, hipStream_t st,
                         hipEvent_t ev0, hipEvent_t ev1) {
  if (splits == 0 || batch == 0) {
    // nothing to launch: the trace events still mark this point of the stream
    hipError_t e = hipSuccess;
    if (ev0 && ev1) {
      e = hipEventRecord(ev0, st);
      if (e == hipSuccess) e = hipEventRecord(ev1, st);
    }
    return e;
  }
  if (dtype == 0) {
    if (D == 128) return launch_decode_t<2, 128>(mode, a, splits, batch, st, ev0, ev1);
    if (D == 64) return launch_decode_t<2, 64>(mode, a, splits, batch, st, ev0, ev1);
  } else if (dtype == 2) {
    if (D == 128) return launch_decode_t<1, 128>(mode, a, splits, batch, st, ev0, ev1);
    if (D == 64) return launch_decode_t<1, 64>(mode, a, splits, batch, st, ev0, ev1);
  } else {
    if (D == 128) return launch_decode_t<4, 128>(mode, a, splits, batch, st, ev0, ev1);
    if (D == 64) return launch_decode_t<4, 64>(mode, a, splits, batch, st, ev0, ev1);
  }
  return hipErrorInvalidValue;
}

template <int ESZ, int D>
static void launch_combine_t(const CombineArgs& a, dim3 grid, hipStream_t st) {
  if (a.s_cap >= 1 && a.s_cap <= 8)
    hipLaunchKernelGGL((combine_kernel<ESZ, D, 8>), grid, dim3(64), 0, st, a);
  else if (a.s_cap >= 1 && a.s_cap <= 16)
    hipLaunchKernelGGL((combine_kernel<ESZ, D, 16>), grid, dim3(64), 0, st, a);
  else if (a.s_cap >= 1 && a.s_cap <= 32)
    hipLaunchKernelGGL((combine_kernel<ESZ, D, 32>), grid, dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((combine_kernel<ESZ, D, 0>), grid, dim3(64), 0, st, a);
}

hipError_t launch_combine(int dtype, int D, const CombineArgs& a, int batch, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  dim3 grid(a.hq, batch);
  if (dtype == 2) dtype = 0;  // fp8 pools: bfloat16 outputs
  if (dtype == 0 && D == 128) launch_combine_t<2, 128>(a, grid, st);
  else if (dtype == 0 && D == 64) launch_combine_t<2, 64>(a, grid, st);
  else if (dtype == 1 && D == 128) launch_combine_t<4, 128>(a, grid, st);
  else if (dtype == 1 && D == 64) launch_combine_t<4, 64>(a, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lak
