/* Host-only exercise of the C ABI's argument validation, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py: every call below is rejected (or is
 * a pure host query) before any HIP call, so it runs without a GPU.  Extreme shapes probe the size
 * arithmetic of the validation and the workspace planner for overflow.  Exit status 0 = every check
 * held; the sanitizers abort on the first finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "twl.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static twl_cache fake_cache(void) {
  twl_cache c;
  memset(&c, 0, sizeof(c));
  void* fake = (void*)(uintptr_t)0x10000;
  c.batch = 1;
  c.num_q_heads = 32;
  c.num_kv_heads = 8;
  c.head_dim = 128;
  c.page_size = 16;
  c.quant_group = 32;
  c.max_pages_per_seq = 2048;
  c.num_phys_pages = 2048;
  c.max_seq_len = 32768;
  c.page_table = (const int32_t*)fake;
  c.seq_lens = (const int32_t*)fake;
  c.k = fake;
  c.v = fake;
  c.k4 = fake;
  c.k4_meta = fake;
  c.kbound = fake;
  c.key_bits = 4;
  return c;
}

int main(void) {
  void* fake = (void*)(uintptr_t)0x10000;
  float* fout = (float*)fake;
  int32_t* fi = (int32_t*)fake;

  /* pure host queries */
  for (int s = 0; s <= 5; ++s) EXPECT(twl_status_str((twl_status)s) != NULL);
  EXPECT(strstr(twl_version(), "gfx950") != NULL);
  EXPECT(twl_keep_pages(2048, 0.25f) == 512);
  EXPECT(twl_keep_pages(0, 0.25f) == 0);
  EXPECT(twl_keep_pages(10, NAN) == -1);
  EXPECT(twl_keep_pages(10, INFINITY) == -1);
  EXPECT(twl_keep_pages(INT32_MAX, 1e30f) == INT32_MAX);
  EXPECT(twl_keep_pages(-5, 0.25f) <= 0);

  twl_cache c = fake_cache();
  size_t a = twl_workspace_bytes(&c, 8192), b = twl_workspace_bytes(&c, 32768);
  EXPECT(a > 0 && b > a && a % 256 == 0);
  EXPECT(twl_workspace_bytes(NULL, 8192) == 0);
  EXPECT(twl_workspace_bytes(&c, -1) == 0);
  EXPECT(twl_workspace_bytes(&c, (int64_t)1 << 40) == 0);  /* beyond the top-p capacity */

  /* shapes at and past the size limits: rejected, never overflowing */
  const int32_t big[] = {1, 2, 1 << 15, 65535, 1 << 24, INT32_MAX};
  for (unsigned i = 0; i < sizeof(big) / sizeof(big[0]); ++i)
    for (unsigned j = 0; j < sizeof(big) / sizeof(big[0]); ++j) {
      twl_cache x = fake_cache();
      x.batch = big[i];
      x.max_pages_per_seq = big[j];
      x.num_phys_pages = big[j];
      x.max_seq_len = big[j] > INT32_MAX / 16 ? INT32_MAX : 16 * big[j];
      (void)twl_workspace_bytes(&x, 65536);
      (void)twl_workspace_bytes(&x, (int64_t)1 << 22);
      twl_decode_params prm = {0.9f, 0.25f, 0.088f, 32, 0, 0};
      twl_status st = twl_decode_noalloc(&x, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, NULL);
      EXPECT(st != TWL_OK);  /* rejected, or (a valid shape) no usable GPU here */
    }
  {
    twl_cache x = fake_cache();
    x.num_kv_heads = 0;
    EXPECT(twl_workspace_bytes(&x, 8192) == 0);
    x = fake_cache();
    x.num_q_heads = 24; /* G = 3 */
    twl_decode_params prm = {0.9f, 0.25f, 0.088f, 32, 0, 0};
    EXPECT(twl_decode(&x, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EUNSUPPORTED);
    x = fake_cache();
    x.head_dim = 64;
    EXPECT(twl_decode(&x, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EUNSUPPORTED);
    x = fake_cache();
    x.max_seq_len = 16 * 2048 + 1;
    EXPECT(twl_decode(&x, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
  }

  /* decode parameters */
  const float bad_p[] = {0.f, -0.1f, 1.0001f, NAN, INFINITY};
  for (unsigned i = 0; i < sizeof(bad_p) / sizeof(bad_p[0]); ++i) {
    twl_decode_params prm = {bad_p[i], 0.25f, 0.088f, 32, 0, 0};
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
  }
  {
    twl_decode_params prm = {0.9f, 0.25f, 0.088f, 0, 0, 0};
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    prm.iters = 65;
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    prm.iters = 32;
    prm.keep_frac = 0.f;
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    prm.keep_frac = 0.25f;
    prm.sm_scale = NAN;
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    prm.sm_scale = 0.088f;
    prm.topk = -1;
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    prm.topk = 0;
    /* misaligned q, missing out, half a CSR, small and misaligned workspaces */
    EXPECT(twl_decode(&c, (char*)fake + 2, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) ==
           TWL_EINVAL);
    EXPECT(twl_decode(&c, fake, &prm, NULL, NULL, NULL, NULL, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, fi, NULL, 0, fake, 1u << 30, NULL) == TWL_EINVAL);
    const size_t need = twl_workspace_bytes(&c, 16 * 512);
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, fake, need - 256, NULL) == TWL_EWORKSPACE);
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, (char*)fake + 16, need, NULL) ==
           TWL_EWORKSPACE);
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, NULL, NULL, 0, NULL, need, NULL) == TWL_EWORKSPACE);
    EXPECT(twl_decode(&c, fake, &prm, fout, NULL, NULL, fi, fi, 8 * 8192 - 1, fake, need, NULL) == TWL_EINVAL);
  }

  /* split entry points */
  EXPECT(twl_quantize_k(&c, NULL, fi, 16, NULL) == TWL_EINVAL);
  EXPECT(twl_quantize_k(&c, fi, fi, -1, NULL) == TWL_EINVAL);
  EXPECT(twl_quantize_k(NULL, fi, fi, 16, NULL) == TWL_EINVAL);
  EXPECT(twl_select_pages(&c, fake, 0.25f, 511, fi, fi, fake, (size_t)1 << 40, NULL) == TWL_EINVAL);
  EXPECT(twl_select_pages(&c, fake, NAN, 512, fi, fi, fake, (size_t)1 << 40, NULL) == TWL_EINVAL);
  {
    twl_candidates both = {fi, fi, fi, 4};
    EXPECT(twl_estimate_topp(&c, fake, 0.088f, 0.9f, 32, &both, fout, NULL, NULL, 0, fi, fi, 1 << 30, fake,
                             (size_t)1 << 40, NULL) == TWL_EINVAL);
    twl_candidates nocount = {fi, NULL, NULL, 4};
    EXPECT(twl_estimate_topp(&c, fake, 0.088f, 0.9f, 32, &nocount, fout, NULL, NULL, 0, fi, fi, 1 << 30, fake,
                             (size_t)1 << 40, NULL) == TWL_EINVAL);
    twl_candidates neg = {fi, NULL, fi, -3};
    EXPECT(twl_estimate_topp(&c, fake, 0.088f, 0.9f, 32, &neg, fout, NULL, NULL, 0, fi, fi, 1 << 30, fake,
                             (size_t)1 << 40, NULL) != TWL_OK);
  }
  EXPECT(twl_sparse_attn(&c, fake, 0.088f, fi, fi, -1, fout, NULL, fake, (size_t)1 << 40, NULL) == TWL_EINVAL);
  EXPECT(twl_select_clusters_topp(&c, fake, 0.088f, 0.0f, 32, fake, fi, fi, 64, fi, fi, fake, (size_t)1 << 40,
                                  NULL) == TWL_EINVAL);
  EXPECT(twl_select_clusters_topp(&c, fake, 0.088f, 0.95f, 32, fake, fi, fi, 65537, fi, fi, fake, (size_t)1 << 40,
                                  NULL) == TWL_EUNSUPPORTED);
  EXPECT(twl_cluster_value_means(&c, fi, fi, 0, fout, NULL) == TWL_EINVAL);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
