/* A plain C99 client of libnbody.so: it includes include/nbody.h and calls
 * the entry points that need no GPU (version, status strings, variant
 * tables, workspace sizes) and the argument checks that every entry point
 * runs before it touches the HIP runtime.  No pointer passed here is ever
 * dereferenced: the checks reject each call first.  Prints "ok" and returns
 * 0, or names the first failed check and returns 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nbody.h"

static int failures = 0;

static void expect(int cond, const char *what) {
  if (!cond) {
    printf("FAILED: %s\n", what);
    ++failures;
  }
}

int main(void) {
  /* plain addresses that are never read: 16-byte aligned and disjoint, a
   * misaligned one, and one that overlaps the first */
  float *const a = (float *)(uintptr_t)0x100000;
  float *const b = (float *)(uintptr_t)0x200000;
  float *const odd = (float *)(uintptr_t)0x300004;
  float *const near_a = (float *)(uintptr_t)0x100010;
  const int64_t n = 1000;
  int v, k, t, w, s, st, u, lg;
  size_t need;

  expect(nbody_abi_version() == NBODY_ABI_VERSION, "abi version");
  expect(strcmp(nbody_status_string(NBODY_OK), "ok") == 0, "status string of NBODY_OK");
  expect(nbody_status_string(NBODY_ERR_HIP) != NULL, "status string of NBODY_ERR_HIP");

  /* the one-sided pass */
  expect(nbody_accel(NULL, n, 1.0f, 1e-4f, b, NULL) == NBODY_ERR_INVALID_ARG, "null posmass");
  expect(nbody_accel(a, -1, 1.0f, 1e-4f, b, NULL) == NBODY_ERR_INVALID_ARG, "negative n");
  expect(nbody_accel(a, NBODY_MAX_N + 1, 1.0f, 1e-4f, b, NULL) == NBODY_ERR_INVALID_ARG,
         "n above NBODY_MAX_N");
  expect(nbody_accel(a, n, 1.0f, 0.0f, b, NULL) == NBODY_ERR_INVALID_ARG, "eps2 = 0");
  expect(nbody_accel(odd, n, 1.0f, 1e-4f, b, NULL) == NBODY_ERR_ALIGNMENT, "misaligned posmass");
  expect(nbody_accel(a, n, 1.0f, 1e-4f, near_a, NULL) == NBODY_ERR_ALIAS, "overlapping output");
  expect(nbody_accel(NULL, 0, 1.0f, 1e-4f, NULL, NULL) == NBODY_OK, "n = 0 is a no-op");
  expect(nbody_accel_variant(a, n, 1.0f, 1e-4f, b, nbody_accel_variant_count(), NULL) ==
             NBODY_ERR_INVALID_ARG,
         "unknown variant");

  /* the variant table */
  v = nbody_accel_variant_for_n(1 << 20);
  expect(v >= 0 && v < nbody_accel_variant_count(), "variant for 2^20 in range");
  expect(nbody_accel_variant_info(v, &k, &t, &w, &s, &st, &u, &lg) == NBODY_OK, "variant info");
  expect(k >= 1 && t >= 1 && w >= 1 && s >= 1 && u >= 1 && lg >= 1 && t % lg == 0,
         "variant info fields");
  expect(nbody_accel_variant_info(-1, NULL, NULL, NULL, NULL, NULL, NULL, NULL) ==
             NBODY_ERR_INVALID_ARG,
         "variant info of -1");

  /* the pair-symmetric pass: workspace sizes and checks */
  need = nbody_accel_symmetric_workspace_bytes((int64_t)1 << 20, -1);
  expect(need == (size_t)6442450944u, "2^20 workspace is 12 N P bytes with 2048-body panels");
  expect(nbody_accel_symmetric_workspace_bytes(0, -1) == 0, "no workspace for n = 0");
  expect(nbody_accel_symmetric(a, n, 1.0f, 1e-4f, b, -1, NULL, 0, NULL) == NBODY_ERR_WORKSPACE,
         "missing workspace");
  expect(nbody_accel_symmetric_chunked_workspace_bytes((int64_t)1 << 20, -1, 0) <
             need / 2,
         "chunked workspace is bounded");

  /* the integrator, the step loop and the energy */
  expect(nbody_leapfrog_step(a, a, b, 1e-3f, n, NULL) == NBODY_ERR_ALIAS, "vel aliases posmass");
  expect(nbody_kdk_run(a, b, near_a, n, 1.0f, 1e-4f, 1e-3f, 1, 0, -1, NULL, 0, NULL) ==
             NBODY_ERR_ALIAS,
         "kdk_run with overlapping arrays");
  expect(nbody_energy_workspace_bytes(0) == 0, "no energy workspace for n = 0");
  expect(nbody_energy(a, b, n, 1.0f, 1e-4f, NULL, 0, (double *)(uintptr_t)0x400000, NULL) ==
             NBODY_ERR_WORKSPACE,
         "energy without workspace");

  /* the launch cap */
  expect(nbody_set_launch_block_cap(-1) == NBODY_ERR_INVALID_ARG, "negative launch cap");
  expect(nbody_set_launch_block_cap(0) == NBODY_OK, "launch cap 0");

  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
