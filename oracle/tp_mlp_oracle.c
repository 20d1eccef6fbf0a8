/*
 * CPU fp64 oracle for the tensor-parallel (Megatron-style) MLP shard forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU kernels.
 *
 * What it computes (the plain definition, in double precision, no blocking,
 * no intermediate rounding):
 *
 *   Given full X[M,H], W[H,F], b[F], V[F,H] and a shard count k dividing F,
 *   with Fk = F/k:
 *   1. shard i owns W_i = W[:, i*Fk:(i+1)*Fk], b_i = b[i*Fk:(i+1)*Fk] and
 *      V_i = V[i*Fk:(i+1)*Fk, :]  (column split of the first linear layer,
 *      row split of the second: "千亿参数模型如何拆分到多张GPU上训练",
 *      张量并行 section, 方案一 / 方案二; "大模型分布式并行策略详解：TP、DP、PP、
 *      CP、EP核心原理与实战" §4.1);
 *   2. A_i = X W_i + b_i  (the ColumnParallelLinear forward, matmul plus the
 *      per-slice bias: "AI大模型分布式训练：张量并行与流水线并行深度实践" §2.1);
 *   3. Y_i = GeLU(A_i), applied per shard with no communication because the
 *      activation is elementwise (方案一 on the first page above), with
 *      GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) = x/2 * erfc(-x / sqrt 2);
 *   4. Z_i = Y_i V_i  (the RowParallelLinear partial product, §2.2 of the
 *      third page above);
 *   5. Z = Z_0 + Z_1 + ... + Z_{k-1}, the all-reduce SUM (§2.2 ibid.; the
 *      identity Z = Y V = Y_1 V_1 + Y_2 V_2, 方案二).
 *
 * All arrays are row-major doubles; the Python wrapper widens bf16/f32 inputs
 * to double exactly before calling.  Sums run in index order.  Parallelism is
 * over output rows only (OpenMP), which does not change any value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* GeLU(x) = x * Phi(x) with the standard normal CDF written as
   Phi(x) = erfc(-x / sqrt 2) / 2, which equals (1 + erf(x / sqrt 2)) / 2 and
   keeps full relative accuracy for negative x, where 1 + erf cancels. */
double oracle_gelu(double x) { return 0.5 * x * erfc(-x / sqrt(2.0)); }

void oracle_gelu_array(const double* x, int64_t n, double* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_gelu(x[i]);
}

/* Step 2 for one row: a[j] = sum_h X[m,h] * W[h, i*Fk + j] + b[i*Fk + j]. */
static void preact_row(const double* X, const double* W, const double* b, int64_t m, int64_t H,
                       int64_t F, int64_t Fk, int64_t i, double* a) {
  const double* x = X + m * H;
  for (int64_t j = 0; j < Fk; ++j) a[j] = 0.0;
  for (int64_t h = 0; h < H; ++h) {
    const double xv = x[h];
    const double* w = W + h * F + i * Fk;
    for (int64_t j = 0; j < Fk; ++j) a[j] += xv * w[j];
  }
  if (b)
    for (int64_t j = 0; j < Fk; ++j) a[j] += b[i * Fk + j];
}

/* Step 4 for one row: z[n] = sum_j y[j] * V[i*Fk + j, n]. */
static void partial_row(const double* y, const double* V, int64_t H, int64_t Fk, int64_t i,
                        double* z) {
  for (int64_t n = 0; n < H; ++n) z[n] = 0.0;
  for (int64_t j = 0; j < Fk; ++j) {
    const double yv = y[j];
    const double* v = V + (i * Fk + j) * H;
    for (int64_t n = 0; n < H; ++n) z[n] += yv * v[n];
  }
}

/* A_i[M,Fk] (pre-activation) of shard i.  b may be NULL (no bias). */
void oracle_col_preact(const double* X, const double* W, const double* b, int64_t M, int64_t H,
                       int64_t F, int k, int i, double* A) {
  const int64_t Fk = F / k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) preact_row(X, W, b, m, H, F, Fk, i, A + m * Fk);
}

/* Y_i[M,Fk] = GeLU(X W_i + b_i) of shard i. */
void oracle_col_gelu(const double* X, const double* W, const double* b, int64_t M, int64_t H,
                     int64_t F, int k, int i, double* Y) {
  const int64_t Fk = F / k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    double* y = Y + m * Fk;
    preact_row(X, W, b, m, H, F, Fk, i, y);
    for (int64_t j = 0; j < Fk; ++j) y[j] = oracle_gelu(y[j]);
  }
}

/* Z_i[M,H] = Y_i[M,Fk] V_i, where V is the full [F,H] matrix and V_i its rows
   [i*Fk, (i+1)*Fk). */
void oracle_row_partial(const double* Yi, const double* V, int64_t M, int64_t F, int64_t H,
                        int k, int i, double* Zi) {
  const int64_t Fk = F / k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) partial_row(Yi + m * Fk, V, H, Fk, i, Zi + m * H);
}

/* Z[n] = parts[0][n] + parts[1][n] + ... + parts[k-1][n], left to right. */
void oracle_shard_reduce(const double* const* parts, int k, int64_t n, double* Z) {
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < n; ++e) {
    double s = 0.0;
    for (int i = 0; i < k; ++i) s += parts[i][e];
    Z[e] = s;
  }
}

/* Whole forward for selected rows of X: Z[r, :] = sum_i GeLU(X[rows[r],:] W_i + b_i) V_i.
   rows == NULL means rows 0..nrows-1.  b may be NULL. */
void oracle_forward_rows(const double* X, const double* W, const double* b, const double* V,
                         int64_t H, int64_t F, int k, const int64_t* rows, int64_t nrows,
                         double* Z) {
  const int64_t Fk = F / k;
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)Fk);
    double* zi = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t m = rows ? rows[r] : r;
      double* z = Z + r * H;
      for (int64_t n = 0; n < H; ++n) z[n] = 0.0;
      for (int i = 0; i < k; ++i) {
        preact_row(X, W, b, m, H, F, Fk, i, y);                 /* step 2 */
        for (int64_t j = 0; j < Fk; ++j) y[j] = oracle_gelu(y[j]); /* step 3 */
        partial_row(y, V, H, Fk, i, zi);                          /* step 4 */
        for (int64_t n = 0; n < H; ++n) z[n] += zi[n];            /* step 5 */
      }
    }
    free(y);
    free(zi);
  }
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
