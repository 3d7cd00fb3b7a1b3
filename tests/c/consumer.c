/* A plain C consumer of include/pisa.h: compiled by gcc as C11 with warnings as errors, linked
 * against libpisa.so, and run by tests/test_c_consumer.py. It calls the host-only entry points
 * (no GPU needed) and prints "consumer ok" when every check holds; otherwise it names the check
 * and exits with status 1. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "pisa.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("check failed at line %d: %s\n", __LINE__, #cond);       \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  pisa_plan_t *plan = NULL;
  pisa_plan_info_t info;
  hipStream_t stream = NULL;

  /* Wan2.1-14B-like 720p layer: N_b = ceil(75600 / 128) = 591, last block 80 rows, k = 60 */
  CHECK(pisa_plan(75600, 40, 128, 128, 0.10, &plan) == PISA_OK);
  CHECK(plan != NULL);
  CHECK(pisa_plan_info(plan, &info) == PISA_OK);
  CHECK(info.L == 75600 && info.H == 40 && info.d == 128 && info.B == 128);
  CHECK(info.n_blocks == 591 && info.n_last == 80 && info.k == 60);
  CHECK(info.dtype == PISA_DTYPE_BF16 && info.routing == PISA_ROUTING_COV);
  CHECK(info.phases == (PISA_PHASE_EXACT | PISA_PHASE_ZEROTH | PISA_PHASE_FIRST));
  CHECK(fabs(info.scale - 1.0 / sqrt(128.0)) < 1e-7);
  CHECK(info.workspace_bytes > 0 && info.workspace_bytes % 256 == 0);

  /* options: valid values accepted, invalid ones refused with a message */
  CHECK(pisa_plan_set(plan, PISA_OPT_ROUTING, PISA_ROUTING_PLAIN) == PISA_OK);
  CHECK(pisa_plan_set(plan, PISA_OPT_PHASES, PISA_PHASE_EXACT | PISA_PHASE_FIRST) == PISA_ERR_INVALID_ARGUMENT);
  CHECK(strlen(pisa_last_error()) > 0);
  CHECK(pisa_plan_set(plan, PISA_OPT_SCALE, -1.0) == PISA_ERR_INVALID_ARGUMENT);
  CHECK(pisa_plan_info(plan, &info) == PISA_OK && info.routing == PISA_ROUTING_PLAIN);

  /* a forward without a workspace is refused before any device use */
  CHECK(pisa_forward(plan, (const void *)0x100000, (const void *)0x200000, (const void *)0x300000,
                     (void *)0x400000, stream) == PISA_ERR_WORKSPACE);

  /* unsupported and invalid plans leave *plan NULL */
  pisa_plan_t *bad = (pisa_plan_t *)&info;
  CHECK(pisa_plan(1000, 2, 96, 128, 0.5, &bad) == PISA_ERR_UNSUPPORTED && bad == NULL);
  CHECK(pisa_plan(1000, 2, 128, 128, 0.0, &bad) == PISA_ERR_INVALID_ARGUMENT && bad == NULL);

  CHECK(strcmp(pisa_status_string(PISA_ERR_DEVICE), "PISA_ERR_DEVICE") == 0);
  CHECK(pisa_plan_destroy(plan) == PISA_OK);
  CHECK(pisa_plan_destroy(plan) == PISA_ERR_INVALID_HANDLE);
  printf("consumer ok\n");
  return 0;
}
