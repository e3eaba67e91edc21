/* A plain C99 caller of libmoe_mi355x.so, built against include/moe.h with
 * -std=c99 -pedantic -Werror by tests/test_abi_cpu.py.  It exercises the
 * entry points that need no device: status strings, the capacity formula and
 * the host-side argument checks, which return before anything is enqueued
 * (so the fake device addresses below are never dereferenced). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;

#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);               \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

int main(void) {
  /* fake, 256-byte aligned device addresses: only the argument checks see them */
  void* P = (void*)(uintptr_t)4096;
  float* PF = (float*)P;
  int32_t* PI = (int32_t*)P;
  void* MIS = (void*)(uintptr_t)(4096 + 8);     /* 8-byte aligned only */
  const moe_status all[] = {MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
                            MOE_ERR_HIP};
  size_t i, j;

  /* every status has its own non-empty name */
  for (i = 0; i < sizeof(all) / sizeof(all[0]); ++i) {
    CHECK(moe_status_string(all[i]) != NULL && moe_status_string(all[i])[0] != '\0');
    for (j = 0; j < i; ++j) CHECK(strcmp(moe_status_string(all[i]), moe_status_string(all[j])) != 0);
  }

  /* capacity: hotelren.com/news/3071227 §2.2's worked example (65536 tokens,
   * 64 experts, factor 1.2: 1228 slots per expert), a factor whose float value
   * lies below the decimal one (1.05: 160 / 8 * 1.05 = 21 exactly), no limit,
   * the cap at T, and the rejected arguments */
  CHECK(moe_capacity(65536, 1, 64, 1.2) == 1228);
  CHECK(moe_capacity(160, 1, 8, 1.05) == 21);
  CHECK(moe_capacity(80, 2, 8, 1.05) == 21);
  CHECK(moe_capacity(40, 2, 8, 0.7) == 7);
  CHECK(moe_capacity(100, 2, 8, 0.0) == 100);
  CHECK(moe_capacity(100, 2, 8, -1.0) == 100);
  CHECK(moe_capacity(100, 2, 2, 4.0) == 100);
  CHECK(moe_capacity(0, 1, 8, 1.0) == -1);
  CHECK(moe_capacity(10, 9, 8, 1.0) == -1);
  CHECK(moe_capacity(10, 0, 8, 1.0) == -1);

  /* workspace sizes are host arithmetic; an unknown op needs none */
  CHECK(moe_workspace_size((moe_op)99, 64, 256, 8, 2, 256, MOE_BF16) == 0);
  (void)moe_workspace_size(MOE_OP_PERMUTE, 64, 256, 8, 2, 256, MOE_BF16);

  /* argument errors, found on the host */
  CHECK(moe_route(NULL, P, NULL, 64, 256, 8, 2, MOE_BF16, PF, PI, PF, PI, NULL, 0, NULL) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_route(P, P, NULL, 64, 256, 8, 9, MOE_BF16, PF, PI, PF, PI, NULL, 0, NULL) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_route(P, P, NULL, 0, 256, 8, 2, MOE_BF16, PF, PI, PF, PI, NULL, 0, NULL) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_route(MIS, P, NULL, 64, 256, 8, 2, MOE_BF16, PF, PI, PF, PI, NULL, 0, NULL) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_route(P, P, NULL, 64, 96, 8, 2, MOE_BF16, PF, PI, PF, PI, NULL, 0, NULL) ==
        MOE_ERR_UNSUPPORTED);
  CHECK(moe_route(P, P, NULL, 64, 256, 300, 2, MOE_BF16, PF, PI, PF, PI, NULL, 0, NULL) ==
        MOE_ERR_UNSUPPORTED);
  CHECK(moe_permute(P, PI, 64, 256, 8, 2, 1.0, MOE_BF16, NULL, PI, PI, PI, PI, P, 1 << 20, NULL) ==
        MOE_ERR_INVALID_ARG);
  CHECK(moe_aux_loss(PF, PI, 64, 8, 9, PF, P, 1 << 20, NULL) == MOE_ERR_INVALID_ARG);
  CHECK(moe_combine(PF, PI, PF, NULL, 0, 64, 256, 2, (moe_dtype)7, P, NULL) ==
        MOE_ERR_UNSUPPORTED);

  printf("c abi check: %d failure(s)\n", failures);
  return failures != 0;
}
