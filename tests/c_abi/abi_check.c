/* A plain C99 caller of the library's C ABI (include/muon.h, include/cautious_adam.h):
 * defaults, plan creation and the host-side validation of both step entry points, with fake
 * device addresses that validation rejects before any HIP call. Prints "abi ok" and exits 0
 * when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "cautious_adam.h"
#include "muon.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

int main(void) {
  muon_config cfg;
  muon_config_default(&cfg);
  CHECK(cfg.ns_steps == 5 && cfg.nesterov == 1 && cfg.row_equalize == 0);
  CHECK(cfg.a > 3.44f && cfg.a < 3.45f && cfg.b < -4.77f && cfg.c > 2.03f);

  /* a plan for the GPT-2 attention / MLP shapes: two padded wide groups */
  const int64_t rows[3] = {768, 3072, 768}, cols[3] = {768, 768, 3072};
  const muon_dtype dts[3] = {MUON_DT_BF16, MUON_DT_BF16, MUON_DT_BF16};
  muon_plan *plan = NULL;
  CHECK(muon_plan_create(&plan, rows, cols, dts, dts, 3, MUON_NS_BF16) == MUON_OK);
  CHECK(plan != NULL);
  const size_t ws = muon_plan_workspace_size(plan);
  CHECK(ws > 0 && ws % 256 == 0);

  /* validation: a NULL gradient is rejected before anything is enqueued */
  muon_matrix mats[3];
  memset(mats, 0, sizeof mats);
  uintptr_t base = (uintptr_t)1 << 40; /* fake device addresses, never dereferenced */
  for (int i = 0; i < 3; ++i) {
    mats[i].param = (void *)(base + (uintptr_t)(4 * i) * (1u << 24));
    mats[i].grad = (const void *)(base + (uintptr_t)(4 * i + 1) * (1u << 24));
    mats[i].momentum = (float *)(base + (uintptr_t)(4 * i + 2) * (1u << 24));
    mats[i].rows = rows[i];
    mats[i].cols = cols[i];
    mats[i].param_dtype = mats[i].grad_dtype = MUON_DT_BF16;
  }
  mats[1].grad = NULL;
  void *wsp = (void *)(base + ((uintptr_t)1 << 30));
  CHECK(muon_step(plan, mats, 3, &cfg, wsp, ws, 0) == MUON_ERR_INVALID_ARG);
  CHECK(strlen(muon_last_error()) > 0);
  CHECK(strcmp(muon_status_string(MUON_ERR_INVALID_ARG), "MUON_ERR_INVALID_ARG") == 0);
  /* a workspace one byte short */
  mats[1].grad = (const void *)(base + (uintptr_t)5 * (1u << 24));
  CHECK(muon_step(plan, mats, 3, &cfg, wsp, ws - 1, 0) == MUON_ERR_WORKSPACE);
  /* the row equaliser needs its state */
  cfg.row_equalize = 1;
  CHECK(muon_step(plan, mats, 3, &cfg, wsp, ws, 0) == MUON_ERR_INVALID_ARG);
  cfg.row_equalize = 0;
  /* concurrency: the stream count is checked before any HIP call; 1 is sequential */
  CHECK(muon_plan_set_concurrency(plan, 0) == MUON_ERR_INVALID_ARG);
  CHECK(muon_plan_set_concurrency(plan, MUON_MAX_STREAMS + 1) == MUON_ERR_INVALID_ARG);
  CHECK(muon_plan_set_concurrency(plan, 1) == MUON_OK);
  CHECK(muon_plan_set_concurrency(NULL, 2) == MUON_ERR_INVALID_ARG);
  muon_plan_destroy(plan);

  /* the static-scratch entry point: a plan larger than its scratch is rejected before any
   * HIP call (24 matrices of 768 x 3072: 245 MiB of workspace), an empty plan is a no-op */
  {
    int64_t br[24], bc[24];
    muon_dtype bd[24];
    for (int i = 0; i < 24; ++i) {
      br[i] = 768;
      bc[i] = 3072;
      bd[i] = MUON_DT_BF16;
    }
    muon_plan *big = NULL;
    CHECK(muon_plan_create(&big, br, bc, bd, bd, 24, MUON_NS_BF16) == MUON_OK);
    CHECK(muon_plan_workspace_size(big) > MUON_STATIC_SCRATCH_BYTES);
    CHECK(muon_step_noalloc(big, NULL, 24, &cfg, 0) == MUON_ERR_WORKSPACE);
    CHECK(strstr(muon_last_error(), "static scratch") != NULL);
    muon_plan_destroy(big);
    muon_plan *none = NULL;
    CHECK(muon_plan_create(&none, NULL, NULL, NULL, NULL, 0, MUON_NS_BF16) == MUON_OK);
    CHECK(muon_step_noalloc(none, NULL, 0, &cfg, 0) == MUON_OK);
    CHECK(muon_step_noalloc(NULL, NULL, 0, &cfg, 0) == MUON_ERR_INVALID_ARG);
    muon_plan_destroy(none);
  }

  /* cautious Adam: defaults and validation */
  muon_adam_config acfg;
  muon_adam_config_default(&acfg);
  CHECK(acfg.step == 1 && acfg.beta1 > 0.89f && acfg.beta2 > 0.998f);
  CHECK(muon_cautious_adam_step(NULL, 0, &acfg, 0) == MUON_OK);
  muon_adam_tensor t;
  memset(&t, 0, sizeof t);
  t.param = (void *)base;
  t.grad = (const void *)(base + 4096);
  t.exp_avg = (float *)(base + 8192);
  t.exp_avg_sq = (float *)(base + 8192); /* aliases exp_avg: rejected */
  t.numel = 256;
  t.wd_mul = 1.0f;
  CHECK(muon_cautious_adam_step(&t, 1, &acfg, 0) == MUON_ERR_INVALID_ARG);
  acfg.step = 0;
  CHECK(muon_cautious_adam_step(&t, 1, &acfg, 0) == MUON_ERR_INVALID_ARG);

  if (failures) return 1;
  printf("abi ok\n");
  return 0;
}
