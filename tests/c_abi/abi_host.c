/* Plain-C user of the MoE library's C ABI: compiles against include/moe.h as
 * C99, links libmoe.so and calls the host-side entry points (sizing,
 * validation, status text) -- none of them touches a GPU.  Prints one line
 * per check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "moe.h"

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond);      \
      return 1;                                                  \
    }                                                            \
    printf("ok %s\n", #cond);                                    \
  } while (0)

int main(void) {
  moe_cfg c;
  memset(&c, 0, sizeof c);
  c.T = 4096;
  c.d = 1024;
  c.E = 8;
  c.k = 2;
  c.f = 4096;
  c.dtype = MOE_BF16;
  c.capacity = moe_capacity(4096, 2, 8, 1.25);
  CHECK(sizeof(moe_cfg) == 64);
  CHECK(c.capacity == 1280);
  CHECK(moe_check_cfg(&c) == MOE_OK);
  CHECK(moe_rows_max(&c) == 8192);
  CHECK(moe_workspace_bytes(&c) > 0);
  CHECK(moe_capacity(100, 2, 4, -1.0) == MOE_NO_CAPACITY);
  c.flags = MOE_FLAG_RECOMPUTE | MOE_FLAG_RENORM | MOE_FLAG_SLOT_PRIORITY |
            MOE_FLAG_DROP_IDENTITY;
  CHECK(moe_check_cfg(&c) == MOE_OK);
  c.flags = 1u << 7;
  CHECK(moe_check_cfg(&c) == MOE_ERR_ARG);
  c.flags = 0;
  c.aux_coeff = -1.0f;
  CHECK(moe_check_cfg(&c) == MOE_ERR_ARG);
  CHECK(moe_workspace_bytes(&c) == 0);
  c.aux_coeff = 0.01f;
  c.k = 9;
  CHECK(moe_check_cfg(&c) == MOE_ERR_ARG);
  c.k = 2;
  /* invalid arguments are rejected before anything is enqueued */
  CHECK(moe_route(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == MOE_ERR_ARG);
  CHECK(strcmp(moe_status_str(MOE_OK), "ok") == 0);
  CHECK(strlen(moe_status_str(MOE_ERR_WORKSPACE)) > 0);
  {
    moe_probe p = {MOE_KERNEL_COUNT_, 0, 0, 0, NULL, NULL};
    c.probe = &p;
    CHECK(moe_check_cfg(&c) == MOE_ERR_ARG);
    p.kernel_id = MOE_KERNEL_GEMM_DH;
    CHECK(moe_check_cfg(&c) == MOE_OK);
    c.probe = NULL;
  }
  printf("all host checks passed\n");
  return 0;
}
