/*
 * c_validate_extremes.c -- gemm_desc_validate over a deterministic grid of
 * extreme descriptions (sizes and strides from 0 to 2^63 - 1, both
 * layouts, both element types, batches), run against the library built
 * with the host AddressSanitizer and UndefinedBehaviorSanitizer (every
 * signed overflow, shift or out-of-bounds access in the checks aborts the
 * run with a report).  Also feeds the plan-taking entry points pointers
 * that are not plans.  Needs no device: validation comes before the device
 * query.  tests/test_abi.py builds and runs it.
 *
 * The plan flags cycle with the grid (none, each tile height, and flag
 * combinations that must be refused: 192-row tiles with the tile consumer,
 * with e4m3 or with both heights); a refused combination that is accepted
 * fails the run.
 *
 * Prints the count of descriptions tried and accepted, and exits 0.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "migemm.h"

static const int64_t kVals[] = {0,
                                1,
                                7,
                                8,
                                255,
                                256,
                                5000,
                                (int64_t)1 << 23,
                                ((int64_t)1 << 23) + 8,
                                (int64_t)1 << 31,
                                (int64_t)1 << 46,
                                (int64_t)1 << 47,
                                ((int64_t)1 << 47) + 16,
                                (int64_t)1 << 59,
                                ((int64_t)1 << 62) + 8,
                                INT64_MAX - 15,
                                INT64_MAX};
enum { kNV = sizeof kVals / sizeof kVals[0] };

static const uint32_t kFlags[] = {0,
                                  MIGEMM_F_TILE_M192,
                                  MIGEMM_F_TILE_M256,
                                  MIGEMM_F_TILE_M192 | MIGEMM_F_TILE_CONSUMER,
                                  MIGEMM_F_TILE_M192 | MIGEMM_F_TILE_M256,
                                  MIGEMM_F_TILE_CONSUMER | MIGEMM_F_TILE_M256,
                                  MIGEMM_F_STREAM_K};
enum { kNF = sizeof kFlags / sizeof kFlags[0] };

int main(void) {
  long tried = 0, accepted = 0, misaccepted = 0;
  for (int dt = 0; dt < 2; ++dt)
    for (int lay = 0; lay < 4; ++lay)
      for (int im = 0; im < kNV; ++im)
        for (int in = 0; in < kNV; in += 2)
          for (int ik = 0; ik < kNV; ik += 3)
            for (int is = 0; is < kNV; ++is) {
              migemm_desc d;
              memset(&d, 0, sizeof d);
              d.M = kVals[im];
              d.N = kVals[in];
              d.K = kVals[ik];
              d.a_type = d.b_type = dt ? MIGEMM_FP8_E4M3 : MIGEMM_BF16;
              d.c_type = d.d_type = MIGEMM_BF16;
              const int64_t ld = kVals[is];
              /* A: row (K-contiguous) or column-major; B likewise. */
              if (lay & 1) d.a_rs = 1, d.a_cs = ld; else d.a_rs = ld, d.a_cs = 1;
              if (lay & 2) d.b_rs = 1, d.b_cs = ld; else d.b_rs = ld, d.b_cs = 1;
              d.c_rs = d.d_rs = ld, d.c_cs = d.d_cs = 1;
              for (int b = 0; b < 3; ++b) {
                d.L = b == 0 ? 1 : (b == 1 ? 3 : INT64_MAX);
                d.a_bs = d.b_bs = d.c_bs = d.d_bs = b == 0 ? 0 : kVals[(is + 3 * b) % kNV];
                d.flags = kFlags[(im + in + ik + is + b + lay) % kNF];
                ++tried;
                if (gemm_desc_validate(&d) == MIGEMM_OK) {
                  ++accepted;
                  const int m192 = (d.flags & MIGEMM_F_TILE_M192) != 0;
                  if (m192 && (dt || (d.flags & (MIGEMM_F_TILE_CONSUMER | MIGEMM_F_TILE_M256))))
                    ++misaccepted;
                }
              }
            }
  /* Pointers that are not plans: refused without being read. */
  static unsigned char junk[4096];
  memset(junk, 0xFF, sizeof junk);
  const migemm_plan* fake = (const migemm_plan*)junk;
  migemm_plan_info info;
  if (gemm_plan_get_info(fake, &info) != MIGEMM_ERR_INVALID_ARG ||
      gemm_run(fake, NULL, NULL, NULL, NULL, 1.0f, 0.0f, NULL, NULL) != MIGEMM_ERR_INVALID_ARG ||
      gemm_plan_workspace_size(fake) != 0 || gemm_plan_destroy((migemm_plan*)junk) != MIGEMM_ERR_INVALID_ARG) {
    printf("a pointer that is not a plan was accepted\n");
    return 1;
  }
  if (misaccepted) {
    printf("%ld refused flag combinations were accepted\n", misaccepted);
    return 1;
  }
  printf("tried %ld accepted %ld\n", tried, accepted);
  return 0;
}
