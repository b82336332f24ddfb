// Host-side checks of the C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code of the library (tests/test_host_sanitizers.py builds and runs it on the CPU).
// Every call here is answered on the host: plans of valid and invalid configurations, and each
// entry point's rejection of bad arguments before anything is launched.  No device is touched.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lh_api.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static lh_config config(int64_t n, int32_t heads, int32_t d, int32_t levels, int32_t pool,
                        int32_t k, int32_t chunk, int32_t mode) {
  lh_config c;
  memset(&c, 0, sizeof(c));
  c.batch = 1;
  c.n_tokens = n;
  c.heads = heads;
  c.head_dim = d;
  c.levels = levels;
  c.pool = pool;
  for (int l = 0; l < LH_MAX_LEVELS; ++l) c.k[l] = k;
  c.chunk = chunk;
  c.dtype = LH_BF16;
  c.select_mode = mode;
  c.softmax_scale = 0.f;
  c.scorer = LH_SCORE_K;
  return c;
}

// S = n_{L-1} + p * sum_{l=1}^{L-1} min(k, n_l) (REFINE) or n_{L-1} + sum_{l=0}^{L-2} min(k, n_l)
static int64_t gathered_length(const lh_config& c) {
  int64_t n[LH_MAX_LEVELS], pw = 1;
  for (int l = 0; l < c.levels; ++l) {
    n[l] = c.n_tokens / pw;
    pw *= c.pool;
  }
  int64_t s = n[c.levels - 1];
  if (c.select_mode == LH_SEL_REFINE) {
    for (int l = 1; l < c.levels; ++l) s += c.pool * (c.k[l] < n[l] ? c.k[l] : n[l]);
  } else {
    for (int l = 0; l + 1 < c.levels; ++l) s += c.k[l] < n[l] ? c.k[l] : n[l];
  }
  return s;
}

static void plans() {
  const lh_config ok[] = {
      config(4096, 2, 64, 3, 4, 128, 64, LH_SEL_REFINE),
      config(524288, 16, 64, 4, 4, 4096, 1024, LH_SEL_REFINE),
      config(1048576, 8, 128, 4, 4, 4096, 1024, LH_SEL_REFINE),
      config(524288, 16, 64, 4, 4, 4096, 1024, LH_SEL_DIRECT),
      config(4096, 2, 64, 8, 2, 20, 64, LH_SEL_REFINE),
      config(16, 2, 64, 2, 4, 1, 16, LH_SEL_REFINE),
      config(2187, 1, 64, 7, 3, 9, 1024, LH_SEL_REFINE),
      config(640, 2, 64, 1, 4, 0, 64, LH_SEL_REFINE),
  };
  for (const lh_config& c : ok) {
    lh_plan_info p;
    memset(&p, 0xA5, sizeof(p));
    EXPECT(lh_plan(&c, &p) == LH_OK);
    EXPECT(p.gathered_len == gathered_length(c));
    EXPECT(p.gathered_pad % 128 == 0 && p.gathered_pad >= p.gathered_len &&
           p.gathered_pad - p.gathered_len < 128);
    EXPECT(p.saved_bytes > 0 && p.ws_backward_bytes > 0);
  }
  lh_config bad = config(4096, 2, 64, 3, 4, 128, 64, LH_SEL_REFINE);
  lh_plan_info p;
  EXPECT(lh_plan(nullptr, &p) == LH_ERR_NULL);
  EXPECT(lh_plan(&bad, nullptr) == LH_ERR_NULL);
  struct Case {
    lh_config c;
    lh_status want;
  };
  Case cases[] = {
      {config(4095, 2, 64, 3, 4, 128, 64, 0), LH_ERR_SHAPE},
      {config(4096, 0, 64, 3, 4, 128, 64, 0), LH_ERR_SHAPE},
      {config(4096, 2, 96, 3, 4, 128, 64, 0), LH_ERR_DTYPE},
      {config(4096, 2, 64, 0, 4, 128, 64, 0), LH_ERR_LEVELS},
      {config(4096, 2, 64, 9, 4, 128, 64, 0), LH_ERR_LEVELS},
      {config(4096, 2, 64, 3, 1, 128, 64, 0), LH_ERR_POOL},
      {config(4096, 2, 64, 3, 17, 128, 64, 0), LH_ERR_POOL},
      {config(4096, 2, 64, 3, 4, -1, 64, 0), LH_ERR_K},
      {config(4096, 2, 64, 3, 4, 128, 48, 0), LH_ERR_CHUNK},
      {config(4096, 2, 64, 3, 4, 128, 4096, 0), LH_ERR_CHUNK},
      {config(12288, 2, 64, 2, 4, 128, 2048, 0), LH_ERR_CHUNK},
      {config(4096, 2, 64, 3, 4, 128, 64, 7), LH_ERR_UNSUPPORTED},
      {config((int64_t(1) << 24) + 1, 1, 64, 1, 4, 0, 64, 0), LH_ERR_SHAPE},
  };
  for (Case& t : cases) EXPECT(lh_plan(&t.c, &p) == t.want);
  lh_config dt = config(4096, 2, 64, 3, 4, 128, 64, 0);
  dt.dtype = 7;
  EXPECT(lh_plan(&dt, &p) == LH_ERR_DTYPE);
  dt = config(4096, 2, 64, 3, 4, 128, 64, 0);
  dt.scorer = 9;
  EXPECT(lh_plan(&dt, &p) == LH_ERR_UNSUPPORTED);
}

static void strings() {
  const lh_status all[] = {LH_OK,         LH_ERR_NULL,      LH_ERR_SHAPE,     LH_ERR_LEVELS,
                           LH_ERR_POOL,   LH_ERR_K,         LH_ERR_CHUNK,     LH_ERR_DTYPE,
                           LH_ERR_ALIGN,  LH_ERR_WORKSPACE, LH_ERR_LAUNCH,    LH_ERR_UNSUPPORTED,
                           LH_ERR_SCRATCH};
  for (lh_status s : all) {
    const char* t = lh_status_string(s);
    EXPECT(t != nullptr && strlen(t) > 0 && strcmp(t, "unknown status") != 0);
  }
  EXPECT(strcmp(lh_status_string(static_cast<lh_status>(12345)), "unknown status") == 0);
}

static void rejections() {
  const lh_config c = config(4096, 2, 64, 3, 4, 128, 64, LH_SEL_REFINE);
  void* ok = reinterpret_cast<void*>(0x10000);   // never dereferenced: validation fails first
  void* bad = reinterpret_cast<void*>(0x10004);  // not 16-byte aligned
  const int32_t* iok = static_cast<const int32_t*>(ok);
  const float* fok = static_cast<const float*>(ok);
  float* fbad = static_cast<float*>(bad);
  lh_stream_t st = nullptr;
  EXPECT(lh_pool_score(nullptr, ok, ok, ok, ok, ok, ok, 0, static_cast<float*>(ok), st) == LH_ERR_NULL);
  EXPECT(lh_pool_score(&c, nullptr, ok, ok, ok, ok, ok, 0, static_cast<float*>(ok), st) == LH_ERR_NULL);
  EXPECT(lh_pool_score(&c, ok, bad, ok, ok, ok, ok, 0, static_cast<float*>(ok), st) == LH_ERR_ALIGN);
  EXPECT(lh_pool_score(&c, ok, ok, ok, ok, ok, ok, 5, static_cast<float*>(ok), st) == LH_ERR_DTYPE);
  EXPECT(lh_topk(&c, nullptr, static_cast<int32_t*>(ok), st) == LH_ERR_NULL);
  EXPECT(lh_pool_score_topk(&c, ok, ok, ok, ok, ok, ok, 0, static_cast<float*>(ok), nullptr, st) ==
         LH_ERR_NULL);
  EXPECT(lh_pool_score_topk(&c, ok, ok, ok, nullptr, ok, nullptr, 0, fbad,
                            static_cast<int32_t*>(ok), st) == LH_ERR_ALIGN);
  EXPECT(lh_build_map(&c, iok, static_cast<int32_t*>(bad), static_cast<int32_t*>(ok), st) ==
         LH_ERR_ALIGN);
  EXPECT(lh_gather(&c, ok, ok, ok, ok, ok, ok, 0, iok, static_cast<int32_t*>(ok),
                   static_cast<int32_t*>(ok), ok, ok, nullptr, st) == LH_ERR_NULL);
  EXPECT(lh_gather(&c, ok, ok, ok, ok, ok, ok, 3, iok, static_cast<int32_t*>(ok),
                   static_cast<int32_t*>(ok), ok, ok, ok, st) == LH_ERR_DTYPE);

  lh_attn_desc d;
  memset(&d, 0, sizeof(d));
  d.batch = 1;
  d.heads = 1;
  d.seq = 100;
  d.head_dim = 64;
  for (int i = 0; i < 3; ++i) {
    const int64_t s[3] = {100 * 64, 100 * 64, 64};
    d.q_stride[i] = d.k_stride[i] = d.v_stride[i] = d.o_stride[i] = s[i];
  }
  d.causal = 1;
  EXPECT(lh_attn_fwd(&d, ok, ok, ok, static_cast<float*>(ok), fbad, st) == LH_ERR_ALIGN);
  size_t nbytes = 0;
  EXPECT(lh_attn_ws_bytes(&d, &nbytes) == LH_OK && nbytes >= 128 * 4);
  EXPECT(lh_attn_bwd(&d, ok, ok, ok, fok, fok, ok, static_cast<float*>(ok), static_cast<float*>(ok),
                     static_cast<float*>(ok), ok, nbytes - 1, st) == LH_ERR_WORKSPACE);
  lh_attn_desc d0 = d;
  d0.seq = 0;
  EXPECT(lh_attn_fwd(&d0, ok, ok, ok, static_cast<float*>(ok), static_cast<float*>(ok), st) ==
         LH_ERR_SHAPE);
  lh_attn_desc d1 = d;
  d1.q_stride[2] = 68;  // rows no longer 16-byte aligned
  EXPECT(lh_attn_fwd(&d1, ok, ok, ok, static_cast<float*>(ok), static_cast<float*>(ok), st) ==
         LH_ERR_ALIGN);
  EXPECT(lh_attn_fwd_mapped(&c, ok, ok, ok, ok, ok, ok, nullptr, static_cast<float*>(ok),
                            static_cast<float*>(ok), st) == LH_ERR_NULL);
  EXPECT(lh_attn_bwd_mapped(&c, ok, ok, ok, ok, ok, ok, iok, fok, fok, ok, static_cast<float*>(ok),
                            static_cast<float*>(ok), static_cast<float*>(ok), 4, st) ==
         LH_ERR_UNSUPPORTED);
  EXPECT(lh_scatter(&c, iok, fok, bad, st) == LH_ERR_ALIGN);
  EXPECT(lh_scatter_bwd(&c, iok, fok, ok, ok, nullptr, st) == LH_ERR_NULL);
  EXPECT(lh_gather_pool_bwd(&c, iok, fok, fok, fok, ok, ok, bad, st) == LH_ERR_ALIGN);

  lh_plan_info p;
  EXPECT(lh_plan(&c, &p) == LH_OK);
  EXPECT(lh_forward(&c, ok, ok, ok, ok, ok, ok, p.ws_forward_bytes - 1, st) == LH_ERR_WORKSPACE);
  EXPECT(lh_forward(&c, ok, ok, ok, nullptr, ok, ok, size_t(1) << 40, st) == LH_ERR_NULL);
  EXPECT(lh_backward(&c, ok, ok, ok, ok, ok, ok, ok, ok, ok, p.ws_backward_bytes - 1, st) ==
         LH_ERR_WORKSPACE);
  EXPECT(lh_backward(&c, nullptr, ok, ok, ok, ok, ok, ok, ok, ok, size_t(1) << 40, st) ==
         LH_ERR_NULL);
  // a forward workspace above the static scratch is refused before any device call
  const lh_config big = config(int64_t(1) << 20, 16, 64, 4, 4, 4096, 1024, LH_SEL_REFINE);
  EXPECT(lh_plan(&big, &p) == LH_OK && p.ws_forward_bytes > LH_NOALLOC_SCRATCH_BYTES);
  EXPECT(lh_forward_noalloc(&big, ok, ok, ok, ok, ok, st) == LH_ERR_SCRATCH);
  EXPECT(lh_forward_noalloc(&c, ok, nullptr, ok, ok, ok, st) == LH_ERR_NULL);
}

int main() {
  plans();
  strings();
  rejections();
  if (failures) {
    fprintf(stderr, "%d host checks failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
