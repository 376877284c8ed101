/*
 * c_client.c -- the C ABI used from plain C, with no Python or PyTorch: the
 * program owns its device memory (hipMalloc) and stream, and calls
 * include/migemm.h directly.  Built by the package's build step into
 * tests/_build/c_client; tests/test_c_client.py runs it on a GPU.
 *
 * Inputs are small integers, so every result is exact and known in closed
 * form: A[i][k] and B[k][j] take values in {-1, 0, 1}, K = 104, so
 * |(A B)[i][j]| <= 104, and with C = 1 and beta = 0.5 each D value is an
 * integer plus 0.5 of magnitude at most 104.5 -- exact in bf16 (8
 * significant bits).  Checked, bit for bit:
 *   1. gemm_run with beta (M, N ragged against the 256 x 256 tiles; K not a
 *      whole number of 64-element stages);
 *   2. a stream-K plan run through gemm_run_no_alloc (its workspace comes
 *      from the library's fixed scratch; no caller allocation);
 *   3. a destroyed plan is refused with MIGEMM_ERR_INVALID_ARG and D is left
 *      as it was.
 * Prints "c_client: OK" and exits 0, or names the first failure and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "migemm.h"

enum { M = 300, N = 264, K = 104 };  /* row pitches 208 and 528 bytes: 16-byte aligned */

static uint16_t bf16_bits(float f) { /* exact for the values used here */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* Entries in {-1, 0, 1}, varying along both dimensions of each operand. */
static int a_val(int i, int k) { return (7 * i + 2 * k) % 3 - 1; }
static int b_val(int k, int j) { return (5 * k + 11 * j + 1) % 3 - 1; }

static float bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "c_client: %s failed: %s\n", #x, hipGetErrorString(e_)); \
      return 1;                                                                \
    }                                                                          \
  } while (0)

#define ST_OK(x)                                                                  \
  do {                                                                            \
    int s_ = (x);                                                                 \
    if (s_ != MIGEMM_OK) {                                                        \
      fprintf(stderr, "c_client: %s gave %s\n", #x, gemm_status_string(s_));      \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

static int check_d(const uint16_t* got, const int32_t* ab, const char* what) {
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < N; ++j) {
      const float want = (float)ab[i * N + j] + 0.5f;
      if (got[i * N + j] != bf16_bits(want)) {
        fprintf(stderr, "c_client: %s: D[%d][%d] = %g, expected %g\n", what, i, j,
                bf16_value(got[i * N + j]), want);
        return 1;
      }
    }
  return 0;
}

int main(void) {
  static uint16_t hA[M * K], hB[K * N], hC[M * N], hD[M * N];
  static int32_t ab[M * N];
  for (int i = 0; i < M; ++i)
    for (int k = 0; k < K; ++k) hA[i * K + k] = bf16_bits((float)(a_val(i, k)));
  for (int k = 0; k < K; ++k)
    for (int j = 0; j < N; ++j) hB[k * N + j] = bf16_bits((float)(b_val(k, j)));
  for (int i = 0; i < M * N; ++i) hC[i] = bf16_bits(1.0f);
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < N; ++j) {
      int32_t s = 0;
      for (int k = 0; k < K; ++k)
        s += a_val(i, k) * b_val(k, j);
      ab[i * N + j] = s;
    }

  int ndev = 0;
  HIP_OK(hipGetDeviceCount(&ndev));
  HIP_OK(hipSetDevice(0));
  void *dA, *dB, *dC, *dD;
  HIP_OK(hipMalloc(&dA, sizeof hA));
  HIP_OK(hipMalloc(&dB, sizeof hB));
  HIP_OK(hipMalloc(&dC, sizeof hC));
  HIP_OK(hipMalloc(&dD, sizeof hD));
  HIP_OK(hipMemcpy(dA, hA, sizeof hA, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dB, hB, sizeof hB, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dC, hC, sizeof hC, hipMemcpyHostToDevice));
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));

  migemm_desc d;
  memset(&d, 0, sizeof d);
  d.M = M, d.N = N, d.K = K;
  d.a_type = d.b_type = d.c_type = d.d_type = MIGEMM_BF16;
  d.a_rs = K, d.a_cs = 1;   /* row-major A */
  d.b_rs = N, d.b_cs = 1;   /* row-major B */
  d.c_rs = N, d.c_cs = 1;
  d.d_rs = N, d.d_cs = 1;
  d.device = 0;
  ST_OK(gemm_desc_validate(&d));

  /* 1. gemm_run with beta. */
  migemm_plan* plan = NULL;
  ST_OK(gemm_plan_create(&d, &plan));
  if (gemm_plan_workspace_size(plan) != 0) {
    fprintf(stderr, "c_client: a whole-tile plan asked for a workspace\n");
    return 1;
  }
  HIP_OK(hipMemset(dD, 0xFF, sizeof hD));
  ST_OK(gemm_run(plan, dA, dB, dC, dD, 1.0f, 0.5f, NULL, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(hD, dD, sizeof hD, hipMemcpyDeviceToHost));
  if (check_d(hD, ab, "gemm_run")) return 1;

  /* 2. stream-K through the no-allocation entry point. */
  migemm_desc dk = d;
  dk.flags = MIGEMM_F_STREAM_K | MIGEMM_F_STREAM_K_FORCE;
  dk.max_workgroups = 64;
  migemm_plan* plan_k = NULL;
  ST_OK(gemm_plan_create(&dk, &plan_k));
  migemm_plan_info info;
  ST_OK(gemm_plan_get_info(plan_k, &info));
  if (info.stream_k_tiles != 4 || gemm_plan_workspace_size(plan_k) == 0) {
    fprintf(stderr, "c_client: expected a stream-K plan over all 4 tiles with a workspace\n");
    return 1;
  }
  HIP_OK(hipMemset(dD, 0xFF, sizeof hD));
  ST_OK(gemm_run_no_alloc(plan_k, dA, dB, dC, dD, 1.0f, 0.5f, stream));
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(hD, dD, sizeof hD, hipMemcpyDeviceToHost));
  if (check_d(hD, ab, "stream-K gemm_run_no_alloc")) return 1;

  /* 3. a destroyed plan is refused before anything is launched. */
  ST_OK(gemm_plan_destroy(plan_k));
  HIP_OK(hipMemset(dD, 0x7F, sizeof hD));
  int st = gemm_run(plan_k, dA, dB, dC, dD, 1.0f, 0.5f, NULL, stream);
  if (st != MIGEMM_ERR_INVALID_ARG) {
    fprintf(stderr, "c_client: a destroyed plan gave %s\n", gemm_status_string(st));
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));
  HIP_OK(hipMemcpy(hD, dD, sizeof hD, hipMemcpyDeviceToHost));
  for (int i = 0; i < M * N; ++i)
    if (hD[i] != 0x7F7F) {
      fprintf(stderr, "c_client: D changed after a refused run\n");
      return 1;
    }

  ST_OK(gemm_plan_destroy(plan));
  HIP_OK(hipStreamDestroy(stream));
  HIP_OK(hipFree(dA));
  HIP_OK(hipFree(dB));
  HIP_OK(hipFree(dC));
  HIP_OK(hipFree(dD));
  printf("c_client: OK\n");
  return 0;
}
