/* Argument checking of the C ABI, run against a host build of the library
 * instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (see
 * test_abi.py).  Every call below is rejected before anything touches a
 * device, so the program needs no GPU.  Exit status 0: every check held. */
#include <stdio.h>
#include <string.h>

#include "favor.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "abi_check: %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main(void) {
  static float buf[64];
  void* p = buf;
  const float* w = buf;
  long long strides[4] = {4096, 1024, 64, 1};

  EXPECT(favor_abi_version() == 1);
  for (int s = 0; s <= 6; ++s) EXPECT(favor_status_string((favor_status)s) != NULL);
  EXPECT(strcmp(favor_status_string((favor_status)99), "unknown status") == 0);
  EXPECT(strcmp(favor_status_string((favor_status)-1), "unknown status") == 0);
  EXPECT(strcmp(favor_kernel_name((favor_kernel)99), "unknown") == 0);

  /* null buffers */
  EXPECT(favor_attn_noncausal(NULL, p, p, w, 1, p, 1, 1, 16, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_attn_causal(p, p, p, NULL, 1, p, 1, 1, 16, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_attn(p, p, p, w, 1, NULL, 1, 1, 16, 64, 256, 1e-6f, 1, FAVOR_F32, p, 0, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_features(NULL, w, 1, buf, 1, 1, 16, 64, 256, FAVOR_F32, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_attn_noalloc(p, NULL, p, w, 1, p, 1, 1, 16, 64, 256, 1e-6f, 0, FAVOR_BF16, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_attn_noncausal_bwd(p, p, p, w, 1, NULL, p, p, p, 1, 1, 16, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) ==
         FAVOR_ERR_NULL);
  EXPECT(favor_attn_causal_bwd(p, p, p, w, 1, p, p, NULL, p, 1, 1, 16, 64, 256, 1e-6f, FAVOR_F32, p, 0, NULL) ==
         FAVOR_ERR_NULL);
  EXPECT(favor_softmax_attn(p, p, NULL, p, 1, 1, 16, 64, 0.125f, 0, FAVOR_BF16, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_draw_projection(1, 1, 256, 64, 1, 1.f, NULL, NULL) == FAVOR_ERR_NULL);
  EXPECT(favor_attn_strided(p, strides, p, strides, NULL, strides, w, 1, p, strides, 1, 1, 16, 64, 64, 256, 1e-6f, 0,
                            FAVOR_FMAP_POSITIVE, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_NULL);

  /* shapes */
  EXPECT(favor_attn_noncausal(p, p, p, w, 1, p, 0, 1, 16, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_SHAPE);
  EXPECT(favor_attn_noncausal(p, p, p, w, 1, p, 1, 1, 0, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_SHAPE);
  EXPECT(favor_attn_noncausal(p, p, p, w, 3, p, 1, 2, 16, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_SHAPE);
  EXPECT(favor_attn_causal(p, p, p, w, 1, p, 256, 256, 64, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_SHAPE);
  EXPECT(favor_attn_causal(p, p, p, w, 1, p, 1, 1, 1 << 22, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) ==
         FAVOR_ERR_SHAPE);
  EXPECT(favor_attn_causal(p, p, p, w, 1, p, 1, 1, -5, 64, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_SHAPE);

  /* unsupported sizes and types */
  EXPECT(favor_attn_noncausal(p, p, p, w, 1, p, 1, 1, 16, 48, 256, 1e-6f, FAVOR_BF16, p, 0, NULL) ==
         FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_attn_noncausal(p, p, p, w, 1, p, 1, 1, 16, 64, 544, 1e-6f, FAVOR_BF16, p, 0, NULL) ==
         FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_attn_noncausal(p, p, p, w, 1, p, 1, 1, 16, 64, 256, 1e-6f, (favor_dtype)7, p, 0, NULL) ==
         FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_features(p, w, 1, buf, 1, 1, 16, 64, 600, FAVOR_F32, NULL) == FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_features_fmap(p, w, 1, buf, 1, 1, 16, 64, 256, (favor_feature_map)9, FAVOR_F32, NULL) ==
         FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_attn_fmap(p, p, p, w, 1, p, 1, 1, 16, 64, 256, 1e-6f, 0, (favor_feature_map)-1, FAVOR_F32, p, 0,
                         NULL) == FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_attn_causal(p, p, p, w, 1, p, 1, 1, 16, 64, 256, 1e-6f, (favor_dtype)-3, p, 0, NULL) ==
         FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_attn_noncausal_bwd(p, p, p, w, 1, p, p, p, p, 1, 1, 16, 64, 256, 1e-6f, (favor_dtype)2, p, 0, NULL) ==
         FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_attn_strided(p, strides, p, strides, p, strides, w, 1, p, strides, 1, 1, 16, 64, 64, 256, 1e-6f, 0,
                            (favor_feature_map)4, FAVOR_BF16, p, 0, NULL) == FAVOR_ERR_UNSUPPORTED);
  EXPECT(favor_softmax_attn(p, p, p, p, 1, 1, 16, 64, 0.125f, 0, (favor_dtype)5, NULL) == FAVOR_ERR_UNSUPPORTED);

  /* workspace sizes for rejected shapes */
  EXPECT(favor_workspace_bytes(0, 1, 16, 64, 256, 0, FAVOR_BF16) == 0);
  EXPECT(favor_workspace_bytes(1, 1, 16, 40, 256, 1, FAVOR_BF16) == 0);
  EXPECT(favor_workspace_bytes(1, 1, 16, 64, 256, 1, (favor_dtype)9) == 0);
  EXPECT(favor_workspace_bytes_fmap(1, 1, 16, 64, 0, 0, FAVOR_FMAP_RELU, FAVOR_F32) == 0);
  EXPECT(favor_workspace_bytes_strided(1, 1, 0, 64, 64, 256, 0, FAVOR_FMAP_POSITIVE, FAVOR_BF16) == 0);
  EXPECT(favor_bwd_workspace_bytes(1, 1, 16, 64, 1000, 0, FAVOR_F32) == 0);

  /* timing API */
  EXPECT(favor_timing_start((favor_kernel)-1, 4) != FAVOR_OK);
  {
    int n = 0;
    EXPECT(favor_timing_stop((favor_kernel)77, NULL, 0, &n) != FAVOR_OK);
  }
  EXPECT(favor_timing_start(FAVOR_KERNEL_CAUSAL, 0) != FAVOR_OK);
  EXPECT(favor_kernel_name(FAVOR_KERNEL_CAUSAL) != NULL);

  if (failures) {
    fprintf(stderr, "abi_check: %d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_check: all checks passed\n");
  return 0;
}
