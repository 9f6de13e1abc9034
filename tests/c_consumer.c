/* A plain C11 consumer of include/gemm_w4a4.h: compiled by gcc and linked
 * against libgemm_w4a4.so by tests/test_c_consumer.py. It uses only the C
 * ABI (no HIP or torch headers) and only calls that need no GPU: the plan,
 * the variant tables, the error strings and argument validation, which
 * returns before any HIP call. Prints one line per check; exit status 0 iff
 * all pass. */
#include <stdio.h>
#include <string.h>

#include "gemm_w4a4.h"

static int failures = 0;

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

int main(void) {
  gemm_w4a4_plan_t pl;
  memset(&pl, 0, sizeof pl);
  check(gemm_w4a4_plan(4096, 3072, 3072, 32, &pl) == GEMM_W4A4_OK, "plan at 4096x3072x3072 R32");
  check(pl.block_m * pl.tiles_m >= 4096 && pl.block_n * pl.tiles_n >= 3072, "plan covers M and N");
  check(pl.grid == pl.tiles_m * pl.tiles_n && pl.k_stages * pl.block_k >= 3072, "grid and k stages");
  check(pl.lds_bytes > 0 && pl.lds_bytes <= pl.lds_limit, "LDS within the limit");
  check(pl.tail_variant == -1 && pl.tail_rows == 0, "4096 rows: one launch");
  check(gemm_w4a4_plan(4352, 3072, 3840, 128, &pl) == GEMM_W4A4_OK && pl.tail_variant >= 0 &&
            pl.block_m * pl.tiles_m + pl.tail_rows == 4352 && pl.block_m % pl.tail_block_m == 0 &&
            pl.tail_splits >= 1 &&
            pl.tail_grid == (pl.tail_rows + pl.tail_block_m - 1) / pl.tail_block_m *
                                ((3072 + pl.tail_block_n - 1) / pl.tail_block_n) * pl.tail_splits,
        "4352 rows: whole tile rows, then a tail launch over the rest");
  check(gemm_w4a4_plan(4096, 3072, 3000, 32, &pl) == GEMM_W4A4_EINVAL, "K % 16 != 0 rejected");
  check(gemm_mxfp4_plan(64, 64, 48, 0, &pl) == GEMM_W4A4_EINVAL, "MXFP4 K % 32 != 0 rejected");

  const int nv = gemm_w4a4_num_variants(), nmx = gemm_mxfp4_num_variants();
  check(nv >= 1 && nmx >= 1, "variant tables are not empty");
  for (int v = 0; v < nv; ++v)
    check(gemm_w4a4_variant_info(v, &pl) == GEMM_W4A4_OK && pl.variant == v, "NVFP4 variant info");
  check(gemm_w4a4_variant_info(nv, &pl) == GEMM_W4A4_EINVAL, "variant index past the table");

  const char* s = gemm_w4a4_strerror(GEMM_W4A4_EALIGN);
  check(s != NULL && strlen(s) > 0, "strerror");

  /* argument validation: no device memory needed, nothing is enqueued */
  const uint8_t* nul = NULL;
  check(gemm_w4a4(nul, nul, nul, nul, NULL, NULL, NULL, NULL, NULL, 16, 16, 32, 0, NULL) ==
            GEMM_W4A4_EINVAL, "NULL operands rejected");
  check(gemm_w4a4((const uint8_t*)16, (const uint8_t*)16, (const uint8_t*)16, (const uint8_t*)16,
                  (const float*)16, (const float*)16, NULL, NULL, (uint16_t*)4096, 0, 16, 32, 0,
                  NULL) == GEMM_W4A4_EINVAL, "M = 0 rejected");
  check(gemm_mxfp4_f16((const uint8_t*)16, (const uint8_t*)16, (const uint8_t*)16,
                       (const uint8_t*)16, (const float*)16, (const float*)16, NULL, NULL,
                       (uint16_t*)4096, 16, 16, 32, GEMM_W4A4_MAX_R + 1, NULL) == GEMM_W4A4_EINVAL,
        "R past the maximum rejected");
  /* the struct sizes, for the Python binding's mirror of them */
  printf("sizeof gemm_w4a4_plan_t %d\n", (int)sizeof(gemm_w4a4_plan_t));
  printf("sizeof quantize_w4a4_plan_t %d\n", (int)sizeof(quantize_w4a4_plan_t));
  return failures == 0 ? 0 : 1;
}
