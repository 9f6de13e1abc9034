// Re-solves one tile instance's LDS budget with the solver of
// bit_quantized_gemm_amd/csrc/w4a4_layout.hpp, host-only. Built by
// tests/test_budget.py with W4A4_LU_ACCOUNTING_FACTOR = 1 (the true count) or
// 2 (the LoRA-up side piece counted twice, the miscount the SVDQuant W4A4 on
// Blackwell page describes in section 7).
//   budget_probe BM BN THREADS STAGE_BYTES OCC POLICY
// prints: depth place ring_bytes side_bytes lds_bytes
#include <stdio.h>
#include <stdlib.h>

#include "w4a4_layout.hpp"

int main(int argc, char** argv) {
  if (argc != 7) return 2;
  const int bm = atoi(argv[1]), bn = atoi(argv[2]), threads = atoi(argv[3]);
  const int stage = atoi(argv[4]), occ = atoi(argv[5]), policy = atoi(argv[6]);
  // the side-region pieces of the tile, as the kernels count them
  const int wb = (2 * bn + threads - 1) / threads * threads * 4, la = bm * 64, lu = 32 * bn * 2;
  const w4a4::Budget b = w4a4::solve_budget(stage, wb, la, lu * W4A4_LU_ACCOUNTING_FACTOR,
                                            w4a4::kLdsLimit / occ, policy);
  printf("%d %d %d %d %d\n", b.depth, b.place, b.ring_bytes, b.side_bytes, b.lds_bytes);
  return 0;
}
