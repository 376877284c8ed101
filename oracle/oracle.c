/*
 * oracle.c -- plain, slow CPU reference for the persistent pipelined GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library.
 *
 * What it computes (all in IEEE binary64, k ascending, one plain dot product
 * per output element):
 *
 *   ref[i][j]   = alpha * sum_k a(i,k) * b(k,j)  +  beta * c(i,j)
 *   absum[i][j] = sum_k |a(i,k) * b(k,j)|
 *
 * The pages fix the shape of the problem (an M x N x K GEMM with separate
 * element types and strides for A, B, C and D, and an epilogue that forms
 * alpha*acc + beta*C; CUTLASS SM90 cooperative kernel header, "Type Aliases"
 * and the consumer warp-group epilogue call).  They do not fix numerics; the
 * accumulation is done here in fp64 so that the result is exact or within a
 * few fp64 ulps of the exact rational value, and the GPU result is checked against it
 * with the tolerance stated next to each config.
 *
 * The beta term is skipped, and C never read, when beta == 0 (the epilogue of
 * the pages loads C only when a source is needed).
 *
 * Element decoding follows the format definitions:
 *   bf16       sign 1 | exponent 8 (bias 127) | fraction 7
 *   e4m3 (OCP "fn")  sign 1 | exponent 4 (bias 7) | fraction 3,
 *              no infinities, S.1111.111 is NaN, largest finite 448.
 *
 * The consumer stage of the tile hand-off (row sum and row max over each
 * 256-wide slice of D, and a bit copy of D) is recomputed from the GPU's own
 * D by orc_tile_rowstats: a sequential fp32 sum in ascending column order and
 * an IEEE maximumNumber, as defined there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 1, ORC_E4M3 = 2 };

/* bf16 bit pattern -> exact value. */
double orc_bf16_value(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 7) & 0xFF;
  int f = bits & 0x7F;
  double v;
  if (e == 0xFF) {
    v = f ? NAN : INFINITY;
  } else if (e == 0) {
    /* subnormal: 2^(1-127) * f/128 */
    v = ldexp((double)f, 1 - 127 - 7);
  } else {
    /* normal: 2^(e-127) * (1 + f/128) */
    v = ldexp((double)(128 + f), e - 127 - 7);
  }
  return sign ? -v : v;
}

/* OCP e4m3 ("fn") bit pattern -> exact value. */
double orc_e4m3_value(uint8_t bits) {
  int sign = bits >> 7;
  int e = (bits >> 3) & 0xF;
  int f = bits & 0x7;
  double v;
  if (e == 0xF && f == 0x7) {
    v = NAN;
  } else if (e == 0) {
    /* subnormal: 2^(1-7) * f/8 */
    v = ldexp((double)f, 1 - 7 - 3);
  } else {
    /* normal: 2^(e-7) * (1 + f/8) */
    v = ldexp((double)(8 + f), e - 7 - 3);
  }
  return sign ? -v : v;
}

/* Element (r, c) of a matrix stored at `base` with row stride rs and column
 * stride cs, both in elements. */
static double elem(int dtype, const void* base, int64_t rs, int64_t cs, int64_t r, int64_t c) {
  int64_t off = r * rs + c * cs;
  if (dtype == ORC_BF16) return orc_bf16_value(((const uint16_t*)base)[off]);
  return orc_e4m3_value(((const uint8_t*)base)[off]);
}

static int valid_type(int t) { return t == ORC_BF16 || t == ORC_E4M3; }

/* The whole M x N result.  A and B are first decoded (exactly) into fp64
 * arrays, A as [M][K] and B as [N][K], so that each dot product walks two
 * contiguous rows; then for every (i, j) a single running sum over
 * k = 0, 1, ..., K-1.  OpenMP splits the rows i among threads; each element's
 * arithmetic is the same whatever the thread count.
 * Returns 0, or -1 on a bad argument. */
int orc_gemm(int64_t M, int64_t N, int64_t K,
             int a_type, const void* A, int64_t a_rs, int64_t a_cs,
             int b_type, const void* B, int64_t b_rs, int64_t b_cs,
             int c_type, const void* C, int64_t c_rs, int64_t c_cs,
             double alpha, double beta,
             double* ref, double* absum, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || !valid_type(a_type) || !valid_type(b_type)) return -1;
  if (beta != 0.0 && (C == NULL || !valid_type(c_type))) return -1;
  if (M == 0 || N == 0) return 0;
  double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
  if (!Ad || !Bd) {
    free(Ad);
    free(Bd);
    return -1;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i)
    for (int64_t k = 0; k < K; ++k) Ad[i * K + k] = elem(a_type, A, a_rs, a_cs, i, k);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < N; ++j)
    for (int64_t k = 0; k < K; ++k) Bd[j * K + k] = elem(b_type, B, b_rs, b_cs, k, j);

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    const double* a = Ad + i * K;
    for (int64_t j = 0; j < N; ++j) {
      const double* b = Bd + j * K;
      double s = 0.0, t = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = a[k] * b[k];
        s += p;
        t += fabs(p);
      }
      double r = alpha * s;
      if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);
      ref[i * N + j] = r;
      absum[i * N + j] = t;
    }
  }
  free(Ad);
  free(Bd);
  return 0;
}

/* The same definition for a list of n chosen entries (rows[e], cols[e]),
 * decoding elements on the fly.  Used where the full product would take too
 * long on the CPU.  Returns 0, or -1 on a bad argument. */
int orc_gemm_entries(int64_t M, int64_t N, int64_t K,
                     int a_type, const void* A, int64_t a_rs, int64_t a_cs,
                     int b_type, const void* B, int64_t b_rs, int64_t b_cs,
                     int c_type, const void* C, int64_t c_rs, int64_t c_cs,
                     double alpha, double beta,
                     const int64_t* rows, const int64_t* cols, int64_t n,
                     double* ref, double* absum, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || !valid_type(a_type) || !valid_type(b_type)) return -1;
  if (beta != 0.0 && (C == NULL || !valid_type(c_type))) return -1;
  for (int64_t e = 0; e < n; ++e)
    if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t e = 0; e < n; ++e) {
    int64_t i = rows[e], j = cols[e];
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = elem(a_type, A, a_rs, a_cs, i, k) * elem(b_type, B, b_rs, b_cs, k, j);
      s += p;
      t += fabs(p);
    }
    double r = alpha * s;
    if (beta != 0.0) r += beta * elem(c_type, C, c_rs, c_cs, i, j);
    ref[e] = r;
    absum[e] = t;
  }
  return 0;
}

/* The larger of two non-NaN floats, with -0 < +0. */
static float max_signed_zero(float a, float b) {
  if (a > b) return a;
  if (b > a) return b;
  return signbit(a) ? b : a; /* equal: only the sign of a zero can differ */
}

/* Consumer-stage recompute from a bf16 D (row stride d_rs, column stride
 * d_cs, in elements).  The hand-off protocol leaves the consumer's work open
 * ("do something with the tile"); the work checked here is a per-row fp32 sum
 * and maximum over each tile_n-wide slice of D, recomputed from the GPU's own
 * D, so it has exactly one correct value.  Its definition, written out:
 *
 *   for every row r and slice t (columns j0 = t*tile_n .. j1-1, with
 *   j1 = min(N, j0 + tile_n); ld = ceil(N / tile_n)):
 *     s = +0.0f;  for j = j0, j0+1, ..., j1-1:  s = fl32(s + x_j)
 *     m = -inf;   for the same j, skipping NaN: m = maximumNumber(m, x_j)
 *     row_sum[r*ld + t] = s,  row_max[r*ld + t] = m
 *
 * where x_j is the bf16 value of D[r][j] widened exactly to fp32.  The sum is
 * the plain sequential fp32 sum in ascending column order, one rounding per
 * addition; the maximum is IEEE 754-2019 maximumNumber, which ignores NaN and
 * orders -0 below +0, so it too has one correct result (-inf when the slice
 * holds no number).
 * Returns 0, or -1 on a bad argument. */
int orc_tile_rowstats(int64_t M, int64_t N, const uint16_t* D, int64_t d_rs, int64_t d_cs,
                      int64_t tile_n, float* row_sum, float* row_max) {
  if (M < 0 || N < 0 || tile_n < 1) return -1;
  int64_t ld = (N + tile_n - 1) / tile_n;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < M; ++r) {
    for (int64_t t = 0; t < ld; ++t) {
      int64_t j0 = t * tile_n;
      int64_t j1 = j0 + tile_n < N ? j0 + tile_n : N;
      volatile float s = 0.0f; /* volatile: one rounding per addition, in order */
      float m = -INFINITY;
      for (int64_t j = j0; j < j1; ++j) {
        float v = (float)orc_bf16_value(D[r * d_rs + j * d_cs]);
        s = s + v;
        if (!isnan(v)) m = max_signed_zero(m, v);
      }
      row_sum[r * ld + t] = s;
      row_max[r * ld + t] = m;
    }
  }
  return 0;
}

/* Threads OpenMP will use by default (for reporting). */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
