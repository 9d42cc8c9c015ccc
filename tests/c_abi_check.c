/* Plain C99 use of the library's C ABI (host calls only, so it runs without a GPU): builds the
 * 800-frame sigma 6 enhanced-SGA plan and checks its sizes against the AVGGT window rule
 * (kept = ceil(37/2) * ceil(37/3) = 247 patches per compressed frame), its workspace layout, the
 * argument checks that come before any device call, and rejected descriptors. */
#include <stdio.h>
#include <string.h>

#include "vggt_attn.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #c,     \
              vggt_attn_last_error());                                        \
      return 1;                                                               \
    }                                                                         \
  } while (0)

int main(void) {
  vggt_attn_plan_t* p = NULL;
  vggt_attn_layout_t lay;
  int64_t n_kv = -1, n_mean = -1, n_diag = -1;
  double flops = 0.0;
  const unsigned enhanced = VGGT_ATTN_REF_DENSE | VGGT_ATTN_DIAG | VGGT_ATTN_MEAN;
  const int64_t T = 800 * (5 + 37 * 37);

  CHECK(vggt_attn_plan(&p, 800, 37, 37, 5, 16, 64, 6, enhanced, VGGT_ATTN_BF16, VGGT_ATTN_FP32) ==
        VGGT_ATTN_OK);
  CHECK(vggt_attn_counts(p, &n_kv, &n_mean, &n_diag, &flops) == VGGT_ATTN_OK);
  /* frame 0 and every special dense, 247 patches of each of the other 799 frames */
  CHECK(n_kv == 800 * 5 + 37 * 37 + 799 * 247);
  CHECK(n_mean == 799);
  CHECK(n_diag == 799 * (37 * 37 - 247));
  CHECK(flops == 4.0 * 64 * 16 * ((double)T * (double)(n_kv + n_mean) + (double)n_diag));
  CHECK(vggt_attn_counts(p, NULL, NULL, NULL, NULL) == VGGT_ATTN_OK);

  memset(&lay, 0, sizeof lay);
  CHECK(vggt_attn_layout(p, &lay) == VGGT_ATTN_OK);
  CHECK(lay.segments == 1 && lay.keys_per_segment == n_kv + n_mean);
  CHECK(lay.segment_rows % 64 == 0 && lay.segment_rows - lay.keys_per_segment < 64);
  CHECK(lay.total_bytes == (int64_t)vggt_attn_workspace_bytes(p));
  CHECK(lay.off_vpack - lay.off_kpack >= (int64_t)16 * lay.segment_rows * 64 * 2);

  /* Pointer checks run before any device call. */
  CHECK(vggt_attn_forward(p, NULL, NULL, NULL, NULL, NULL, 0, NULL) == VGGT_ATTN_EINVAL);
  CHECK(strlen(vggt_attn_last_error()) > 0);
  CHECK(vggt_attn_forward_sized(p, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == VGGT_ATTN_EINVAL);
  vggt_attn_plan_destroy(p);

  /* Rejected descriptors leave *out NULL. */
  p = (vggt_attn_plan_t*)&lay;
  CHECK(vggt_attn_plan(&p, 4, 8, 8, 5, 2, 64, 3, 0, VGGT_ATTN_BF16, VGGT_ATTN_FP32) == VGGT_ATTN_EINVAL);
  CHECK(p == NULL);
  CHECK(vggt_attn_plan(&p, 4, 8, 8, 5, 2, 128, 1, 0, VGGT_ATTN_BF16, VGGT_ATTN_FP32) ==
        VGGT_ATTN_EUNSUPPORTED);
  CHECK(vggt_attn_plan(&p, 4, 8, 8, 5, 2, 64, 4, VGGT_ATTN_G2F, VGGT_ATTN_BF16, VGGT_ATTN_FP32) ==
        VGGT_ATTN_EINVAL);
  CHECK(vggt_attn_plan(&p, 4, 8, 8, 5, 2, 64, 1, 0, VGGT_ATTN_FP32, VGGT_ATTN_BF16) == VGGT_ATTN_EINVAL);
  CHECK(vggt_attn_plan(NULL, 4, 8, 8, 5, 2, 64, 1, 0, VGGT_ATTN_BF16, VGGT_ATTN_FP32) == VGGT_ATTN_EINVAL);
  CHECK(vggt_attn_workspace_bytes(NULL) == 0);
  vggt_attn_plan_destroy(NULL);

  /* G2F: one segment of L keys per frame. */
  CHECK(vggt_attn_plan(&p, 3, 37, 37, 5, 2, 64, 1, VGGT_ATTN_G2F, VGGT_ATTN_FP32, VGGT_ATTN_FP32) ==
        VGGT_ATTN_OK);
  CHECK(vggt_attn_counts(p, &n_kv, &n_mean, &n_diag, NULL) == VGGT_ATTN_OK);
  CHECK(n_kv == 5 + 37 * 37 && n_mean == 0 && n_diag == 0);
  CHECK(vggt_attn_layout(p, &lay) == VGGT_ATTN_OK && lay.segments == 3 && lay.segment_rows == 1408);
  vggt_attn_plan_destroy(p);

  printf("c abi ok\n");
  return 0;
}
