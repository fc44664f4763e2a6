// Host-side exercise of the C ABI for the sanitizer build: the page allocator, argument
// validation and error paths on metadata-only caches (no device is touched).  Built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the library
// by tests/test_sanitize_host.py; exits non-zero on the first failed expectation.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lak.h"

static int g_fail = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      g_fail = 1;                                                         \
    }                                                                     \
  } while (0)

static lak_cache_desc desc(int layers, int max_batch, int hq, int hkv, int d, int page, int max_pages,
                           int dtype, long long num_pages) {
  lak_cache_desc x;
  std::memset(&x, 0, sizeof(x));
  x.num_layers = layers;
  x.max_batch = max_batch;
  x.num_q_heads = hq;
  x.num_kv_heads = hkv;
  x.head_dim = d;
  x.page_size = page;
  x.max_pages_per_seq = max_pages;
  x.dtype = dtype;
  x.num_pages = num_pages;
  return x;  // pools, page table and lengths NULL: metadata-only
}

static std::vector<int32_t> pages_of(lak_cache* c, int b) {
  std::vector<int32_t> v(4096);
  int32_t n = 0;
  EXPECT(lak_page_table_host(c, b, v.data(), (int32_t)v.size(), &n) == LAK_OK);
  v.resize(n > 0 ? n : 0);
  return v;
}

int main() {
  // --- descriptor validation
  lak_cache* c = nullptr;
  lak_cache_desc d = desc(2, 4, 8, 2, 64, 16, 16, LAK_BF16, 64);
  EXPECT(lak_cache_create(nullptr, &c) == LAK_EINVAL);
  EXPECT(lak_cache_create(&d, nullptr) == LAK_EINVAL);
  lak_cache_desc bad = d;
  bad.num_q_heads = 7;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EINVAL);
  bad = d;
  bad.num_q_heads = 34;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EUNSUPPORTED);
  bad = d;
  bad.head_dim = 96;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EUNSUPPORTED);
  bad = d;
  bad.page_size = 48;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EUNSUPPORTED);
  bad = d;
  bad.dtype = 9;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EINVAL);
  bad = d;
  bad.num_pages = 0;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EINVAL);
  bad = d;
  bad.max_pages_per_seq = 0x7FFFFFFF;
  EXPECT(lak_cache_create(&bad, &c) == LAK_EINVAL);
  EXPECT(std::strlen(lak_last_error()) > 0);
  EXPECT(lak_pool_bytes(&d) == 64LL * 2 * 16 * 64 * 2);
  lak_cache_desc f8 = desc(1, 1, 4, 4, 128, 16, 8, LAK_FP8_E4M3, 5);
  EXPECT(lak_pool_bytes(&f8) == 5LL * 4 * 16 * 128 + 5LL * 4 * 16 * 4);
  EXPECT(lak_pool_bytes(nullptr) == -1);

  // --- allocator on a metadata-only cache
  EXPECT(lak_cache_create(&d, &c) == LAK_OK);
  EXPECT(lak_step_begin(c, nullptr) == LAK_ESTATE);  // no batch yet
  EXPECT(lak_workspace_bytes(c) > 0 && lak_workspace_bytes(c) % 256 == 0);
  const int32_t lens[4] = {0, 15, 16, 17};
  EXPECT(lak_seq_reset(c, 4, lens, 0, nullptr) == LAK_OK);
  EXPECT(lak_free_pages(c) == 64 - (0 + 1 + 1 + 2));
  {
    std::vector<int32_t> seen;
    for (int b = 0; b < 4; ++b)
      for (int32_t p : pages_of(c, b)) {
        EXPECT(p >= 0 && p < 64);
        for (int32_t q : seen) EXPECT(p != q);
        seen.push_back(p);
      }
  }
  for (int s = 0; s < 40; ++s) EXPECT(lak_step_begin(c, nullptr) == LAK_OK);
  {
    int32_t out[4], n = 0;
    EXPECT(lak_seq_lens_host(c, out, 4, &n) == LAK_OK && n == 4);
    for (int b = 0; b < 4; ++b) {
      EXPECT(out[b] == lens[b] + 40);
      EXPECT((int)pages_of(c, b).size() == (out[b] + 15) / 16);
    }
    EXPECT(lak_seq_lens_host(c, out, 3, &n) == LAK_EINVAL);  // cap < batch
  }
  EXPECT(lak_page_table_host(c, 7, nullptr, 0, nullptr) == LAK_EINVAL);
  // run a sequence up to max_pages_per_seq: the next step is refused, lengths unchanged
  const int32_t one[1] = {16 * 16 - 1};
  EXPECT(lak_seq_reset(c, 1, one, 0, nullptr) == LAK_OK);
  EXPECT(lak_step_begin(c, nullptr) == LAK_OK);   // 256 tokens: 16 pages
  EXPECT(lak_step_begin(c, nullptr) == LAK_EINVAL);
  {
    int32_t out[1], n = 0;
    EXPECT(lak_seq_lens_host(c, out, 1, &n) == LAK_OK && out[0] == 256);
  }
  // a batch that needs more pages than the pool holds: ENOPAGE, no active batch after
  const int32_t big[4] = {256, 256, 256, 256};
  const int32_t bigger[4] = {256, 256, 256, 257};
  EXPECT(lak_seq_reset(c, 4, big, 0, nullptr) == LAK_OK);  // exactly 64 pages
  EXPECT(lak_free_pages(c) == 0);
  EXPECT(lak_seq_reset(c, 4, bigger, 0, nullptr) == LAK_EINVAL);  // 17 pages > max_pages_per_seq
  lak_cache_desc dd = desc(1, 4, 8, 2, 64, 16, 64, LAK_BF16, 64);
  lak_cache* c2 = nullptr;
  EXPECT(lak_cache_create(&dd, &c2) == LAK_OK);
  EXPECT(lak_seq_reset(c2, 4, bigger, 0, nullptr) == LAK_ENOPAGE);
  EXPECT(lak_step_begin(c2, nullptr) == LAK_ESTATE);
  // ENOPAGE in a step: all lengths unchanged
  const int32_t full16[4] = {16, 16, 16, 16 * 60};
  EXPECT(lak_seq_reset(c2, 4, full16, 0, nullptr) == LAK_OK);  // 1 + 1 + 1 + 60 = 63 pages
  EXPECT(lak_step_begin(c2, nullptr) == LAK_ENOPAGE);         // four new pages wanted, one free
  {
    int32_t out[4], n = 0;
    EXPECT(lak_seq_lens_host(c2, out, 4, &n) == LAK_OK);
    for (int b = 0; b < 4; ++b) EXPECT(out[b] == full16[b]);
  }
  EXPECT(lak_seq_reset(c2, 0, nullptr, 0, nullptr) == LAK_OK);  // empty batch
  EXPECT(lak_step_begin(c2, nullptr) == LAK_OK);
  EXPECT(lak_seq_reset(c2, 5, lens, 0, nullptr) == LAK_EINVAL);   // above max_batch
  EXPECT(lak_seq_reset(c2, 1, nullptr, 0, nullptr) == LAK_EINVAL);
  const int32_t neg[1] = {-1};
  EXPECT(lak_seq_reset(c2, 1, neg, 0, nullptr) == LAK_EINVAL);
  EXPECT(lak_seq_reset(c2, 1, lens + 1, -1, nullptr) == LAK_EINVAL);
  // pre-reserved pages: steps inside the reservation take no new page
  EXPECT(lak_seq_reset(c2, 1, lens + 1, 40, nullptr) == LAK_OK);  // 15 + 40 tokens: 4 pages
  const long long free0 = lak_free_pages(c2);
  for (int s = 0; s < 49; ++s) EXPECT(lak_step_begin(c2, nullptr) == LAK_OK);  // 64 tokens: still 4 pages
  EXPECT(lak_free_pages(c2) == free0);
  EXPECT(lak_step_begin(c2, nullptr) == LAK_OK);  // the 65th token opens a fifth page
  EXPECT(lak_free_pages(c2) == free0 - 1);

  // --- attention and KV calls on a metadata-only cache fail cleanly (no device buffers)
  int dummy = 0;
  void* p = &dummy;
  EXPECT(lak_seq_reset(c, 4, lens, 0, nullptr) == LAK_OK);
  EXPECT(lak_kv_append(c, 0, p, p, nullptr) == LAK_ESTATE);
  EXPECT(lak_kv_prefill(c, 0, p, p, 64, nullptr) == LAK_ESTATE);
  EXPECT(lak_attn_full(c, 0, p, nullptr, nullptr, 0.1f, p, nullptr, p, 1 << 20, nullptr) == LAK_ESTATE);
  EXPECT(lak_attn_delta_select(c, 0, p, nullptr, nullptr, 0.1f, p, nullptr, 4, 2, LAK_AGG_MAX, LAK_SCOPE_GROUP,
                               (int32_t*)p, (int32_t*)p, 6, nullptr, p, 1 << 20, nullptr) == LAK_ESTATE);
  EXPECT(lak_attn_sparse(c, 0, p, nullptr, nullptr, 0.1f, (int32_t*)p, (int32_t*)p, 6, LAK_SCOPE_GROUP, p, nullptr,
                         p, 1 << 20, nullptr) == LAK_ESTATE);
  EXPECT(lak_attn_sparse_noalloc(c, 0, p, nullptr, nullptr, 0.1f, (int32_t*)p, (int32_t*)p, 6, LAK_SCOPE_GROUP, p,
                                 nullptr, nullptr) == LAK_ESTATE);
  EXPECT(lak_page_select(c, (const float*)p, LAK_SCOPE_GROUP, 4, 2, (int32_t*)p, (int32_t*)p, 6, nullptr) ==
         LAK_ESTATE);
  EXPECT(lak_kv_gather(c, 0, 0, 0, 0, 1, p, p, nullptr) == LAK_ESTATE);
  EXPECT(lak_attn_full(nullptr, 0, p, nullptr, nullptr, 0.1f, p, nullptr, p, 1, nullptr) == LAK_EINVAL);
  lak_stack_step_desc sd;
  std::memset(&sd, 0, sizeof(sd));
  EXPECT(lak_stack_step(c, &sd, p, 1 << 20, nullptr) == LAK_ESTATE);
  EXPECT(lak_trace_decode(c, p, nullptr) == LAK_EINVAL);
  EXPECT(lak_trace_decode(c, nullptr, nullptr) == LAK_OK);
  EXPECT(lak_trace_decode(nullptr, nullptr, nullptr) == LAK_EINVAL);

  // --- many caches of every supported shape, reset and stepped, then destroyed
  const int ds[2] = {64, 128}, ps[3] = {16, 32, 64}, gs[5] = {1, 2, 4, 7, 16};
  for (int di = 0; di < 2; ++di)
    for (int pi = 0; pi < 3; ++pi)
      for (int gi = 0; gi < 5; ++gi)
        for (int dt = 0; dt < 3; ++dt) {
          lak_cache_desc x = desc(3, 5, 2 * gs[gi], 2, ds[di], ps[pi], 40, dt, 200);
          lak_cache* h = nullptr;
          EXPECT(lak_cache_create(&x, &h) == LAK_OK);
          const int32_t ln[5] = {1, ps[pi] - 1, ps[pi], ps[pi] + 1, 7 * ps[pi]};
          EXPECT(lak_seq_reset(h, 5, ln, 3, nullptr) == LAK_OK);
          for (int s = 0; s < 2 * ps[pi]; ++s) EXPECT(lak_step_begin(h, nullptr) == LAK_OK);
          EXPECT(lak_workspace_bytes(h) > 0);
          EXPECT(lak_cache_destroy(h) == LAK_OK);
        }
  EXPECT(lak_cache_destroy(c2) == LAK_OK);
  EXPECT(lak_cache_destroy(c) == LAK_OK);
  EXPECT(lak_cache_destroy(nullptr) == LAK_OK);
  if (g_fail) return 1;
  std::printf("abi host check ok\n");
  return 0;
}
