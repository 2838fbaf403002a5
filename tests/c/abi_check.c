/* Host-only use of libmuon from plain C99 (no GPU call): the header compiles
 * as C, and the plan, query and error paths behave as documented.  Prints one
 * line per check; the Python test compares them with the numpy reference's
 * planner. */
#include <stdio.h>
#include <string.h>

#include "libmuon.h"

int main(void) {
  /* a split QKV-like weight, a tall unit, an fp32 unit, an AdamW vector */
  const muon_param_shape table[4] = {
      {MUON_KIND_MUON, MUON_BF16, 2304, 768, 768, 0},
      {MUON_KIND_MUON, MUON_BF16, 3072, 768, 0, 0},
      {MUON_KIND_MUON, MUON_F32, 300, 701, 0, 0},
      {MUON_KIND_ADAMW, MUON_BF16, 1, 768, 0, 0}};
  muon_plan* plan = NULL;
  muon_plan_options opts = {MUON_NS_STANDARD, -1};
  if (muon_plan_create(table, 4, &opts, &plan) != MUON_OK || !plan) return 1;

  size_t len = 0;
  if (muon_plan_buckets(plan, NULL, 0, &len) != MUON_OK) return 2;
  int32_t buckets[64];
  if (len > 64 || muon_plan_buckets(plan, buckets, 64, &len) != MUON_OK) return 3;
  for (size_t b = 0; b < len / 8; ++b) {
    printf("bucket");
    for (int j = 0; j < 8; ++j) printf(" %d", (int)buckets[8 * b + j]);
    printf("\n");
  }
  /* a capacity below the need writes nothing and says so */
  if (muon_plan_buckets(plan, buckets, 1, &len) != MUON_E_CAPACITY) return 4;

  int64_t units[6 * 16];
  if (muon_plan_units(plan, units, 6 * 16, &len) != MUON_OK) return 5;
  for (size_t u = 0; u < len / 6; ++u) {
    printf("unit");
    for (int j = 0; j < 6; ++j) printf(" %lld", (long long)units[6 * u + j]);
    printf("\n");
  }
  size_t ws = 0;
  if (muon_plan_workspace_bytes(plan, &ws) != MUON_OK || ws == 0) return 6;
  printf("workspace_nonzero 1\n");
  muon_plan_destroy(plan);

  /* argument errors are reported before any device work */
  if (muon_plan_create(table, 4, NULL, NULL) != MUON_E_ARG) return 7;
  muon_param_shape bad = table[0];
  bad.split_rows = 700;
  if (muon_plan_create(&bad, 1, NULL, &plan) != MUON_E_SHAPE || plan) return 8;
  opts.ns_method = 9;
  if (muon_plan_create(table, 4, &opts, &plan) != MUON_E_METHOD) return 9;

  float coeffs[3 * 10];
  if (muon_ns_coefficients(MUON_COEFF_HYBRID, 10, coeffs, 30) != MUON_OK) return 10;
  printf("hybrid_last %.4f %.4f %.4f\n", coeffs[27], coeffs[28], coeffs[29]);
  if (muon_ns_coefficients(MUON_COEFF_QUINTIC, 5, coeffs, 14) != MUON_E_CAPACITY) return 11;

  size_t nb = 0;
  if (ns_orthogonalize_workspace_bytes(1024, 4096, MUON_BF16, MUON_NS_STANDARD, &nb) != MUON_OK) return 12;
  printf("ns_workspace_fits_noalloc %d\n", nb <= (size_t)MUON_NOALLOC_SCRATCH_BYTES);
  if (ns_orthogonalize_noalloc(NULL, 4096, 4096, 4096, MUON_BF16, 5, NULL, MUON_NS_STANDARD, NULL) !=
      MUON_E_WORKSPACE)
    return 13; /* too large for the library's array: rejected before anything else */
  printf("status %s\n", muon_status_string(MUON_E_WORKSPACE));
  printf("version_ok %d\n", muon_version() >= 100);
  return 0;
}
