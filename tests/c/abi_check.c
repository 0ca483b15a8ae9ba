/*
 * A plain C99 consumer of include/xr.h: it compiles against the header alone, links
 * against libxr.so and checks, without a GPU, that the library reports its version and
 * status strings and rejects invalid arguments before touching a device.
 * Exit status 0 on success; the first failed check is printed.
 */
#include <stdio.h>
#include <string.h>

#include "xr.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  void* p = (void*)0x10000;
  void* q = (void*)0x20000;
  float* f = (float*)0x30000;
  int64_t* t = (int64_t*)0x40000;
  CHECK(xr_version() >= 10400);
  CHECK(strcmp(xr_status_string(XR_OK), "ok") == 0);
  CHECK(xr_softmax_fwd(p, 10, q, 10, 4, 10, (xr_dtype_t)7, NULL) == XR_ERR_DTYPE);
  CHECK(xr_softmax_fwd(p, 9, q, 10, 4, 10, XR_F32, NULL) == XR_ERR_STRIDE);
  CHECK(xr_softmax_fwd(p, 10, q, 10, 0, 10, XR_F32, NULL) == XR_OK);
  CHECK(xr_softmax_bwd(p, 8, q, 8, NULL, 8, 2, 8, XR_F32, NULL) == XR_ERR_NULL);
  CHECK(xr_softmax_fwd_ex(p, 10, q, 10, 4, 10, XR_F32, (void*)0x50004, 4096, NULL) ==
        XR_ERR_ALIGN);
  CHECK(xr_softmax_bwd_ex(p, 8, q, 8, NULL, 8, 2, 8, XR_F32, NULL, 0, NULL) == XR_ERR_NULL);
  CHECK(xr_softmax_workspace_bytes(4, 0, XR_F32) == 0);
  CHECK(xr_xent_fwd_bwd(p, 8, t, -1, 8, -100, XR_BF16, f, f, NULL, q, 4096, NULL) == XR_ERR_SHAPE);
  CHECK(xr_xent_fwd_bwd_ex(p, 8, t, 2, 8, -100, XR_BF16, (xr_reduction_t)5, NULL, 0, f, f, NULL,
                           q, 4096, NULL) == XR_ERR_VALUE);
  /* a written buffer inside the logits; row_loss NULL with the none reduction */
  CHECK(xr_xent_fwd_bwd_ex(p, 8, t, 2, 8, -100, XR_BF16, XR_REDUCTION_MEAN, NULL, 0,
                           (float*)((char*)p + 8), f, NULL, q, 4096, NULL) == XR_ERR_ALIAS);
  CHECK(xr_xent_fwd_bwd_ex(p, 8, t, 2, 8, -100, XR_BF16, XR_REDUCTION_MEAN, NULL, 0, f, f, NULL,
                           (char*)p + 16, 4096, NULL) == XR_ERR_ALIAS);
  CHECK(xr_xent_fwd_bwd_ex(p, 8, t, 2, 8, -100, XR_BF16, XR_REDUCTION_NONE, NULL, 0, NULL, NULL,
                           NULL, q, 4096, NULL) == XR_ERR_NULL);
  CHECK(xr_workspace_status(q, 4096, NULL, NULL) == XR_ERR_NULL);
  CHECK(xr_workspace_status(q, 64, (int32_t*)f, NULL) == XR_ERR_WORKSPACE);
  CHECK(xr_probe_copy(q, (char*)q + 16, NULL, 4096, 8, 256, NULL) == XR_ERR_ALIAS);
  CHECK(xr_probe_copy(q, p, NULL, 4096, 8, 100, NULL) == XR_ERR_SHAPE);
  CHECK(xr_probe_copy(q, p, p, 4096, 0, 256, NULL) == XR_ERR_VALUE);
  CHECK(xr_probe_copy(q, q, NULL, 4096, 0, 256, NULL) == XR_ERR_ALIAS);
  CHECK(xr_probe_copy(q, q, p, 4096, 8, 256, NULL) == XR_ERR_VALUE);
  /* operands spanning 2^48 bytes or more */
  CHECK(xr_softmax_fwd(p, (int64_t)1 << 24, q, (int64_t)1 << 24, (int64_t)1 << 24,
                       (int64_t)1 << 24, XR_BF16, NULL) == XR_ERR_SHAPE);
  CHECK(xr_element_mul(p, 8, 4, 8, XR_F32, f, (int64_t)1 << 50, NULL) == XR_ERR_SHAPE);
  CHECK(xr_probe_copy(q, p, NULL, (int64_t)1 << 48, 8, 256, NULL) == XR_ERR_SHAPE);
  CHECK(xr_element_mul(p, 8, 4, 8, XR_F32, NULL, 0, NULL) == XR_ERR_NULL);
  CHECK(xr_nll_fwd(p, 8, q, 8, NULL, f, 4, 8, XR_F32, NULL, 0, NULL) == XR_ERR_NULL);
  CHECK(xr_layernorm_fwd(p, 8, q, 8, q, q, f, f, 4, 8, -1.0f, XR_F32, NULL) == XR_ERR_VALUE);
  CHECK(xr_layernorm_bwd(p, 8, q, 8, q, 8, q, f, f, NULL, q, 4, 8, XR_F32, q, 1 << 20, NULL) ==
        XR_ERR_NULL);
  CHECK(xr_bsr_softmax_bwd(p, 4096, q, 4096, 2, (const int32_t*)t, 20, 4, 4, 48, 1.0f, XR_F32,
                           NULL) == XR_ERR_SHAPE);
  CHECK(xr_plan(9, 4, 8, XR_F32, 1, NULL) == XR_ERR_NULL);
  CHECK(xr_set_option((xr_option_t)99, 0) == XR_ERR_OPTION);
  CHECK(xr_set_profile_events(p, NULL) == XR_ERR_NULL);
  printf("ok\n");
  return 0;
}
