/*
 * CPU fp64 oracle for the tensor-parallel (Megatron-style) MLP shard forward
 * and its backward pass.
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
 * The backward (the gradients of the same block for a loss L, given dZ =
 * dL/dZ; the backward exchange mirrors the forward one:
 * "大模型分布式训练四维并行：DDP、ZeRO、张量、流水线与上下文" §4.3, and forward and
 * backward each take one all-reduce per MLP: "AI大模型分布式训练：张量并行与流水线
 * 并行深度实践" §2.4), by the chain rule through steps 5 .. 2:
 *   6. every shard receives the same dZ (the forward SUM is linear, so
 *      dL/dZ_i = dZ);
 *   7. dY_i = dZ V_i^T and dV_i = Y_i^T dZ  (step 4);
 *   8. dA_i = dY_i * GeLU'(A_i) element-wise, with
 *      GeLU'(x) = Phi(x) + x phi(x), phi(x) = exp(-x^2/2) / sqrt(2 pi)  (step 3);
 *   9. dW_i = X^T dA_i, db_i[j] = sum_m dA_i[m, j], dX_i = dA_i W_i^T  (step 2);
 *  10. dX = dX_0 + ... + dX_{k-1}: X feeds every shard, so its gradient is the
 *      sum over shards (the backward all-reduce).
 *
 * Sequence parallelism (Megatron's split of the block's non-TP region along
 * the sequence, "AI大模型分布式训练：张量并行与流水线并行深度实践" §4.2, with
 * LayerNorm/Dropout sharded along the sequence: "大模型分布式训练四维并行：DDP、
 * ZeRO、张量、流水线与上下文" §4.3):
 *  11. the all-reduce of step 5 is a reduce-scatter followed by an all-gather
 *      (the ring decomposition, §2.1 of that page); under sequence
 *      parallelism each of the k ranks keeps only its reduce-scatter block,
 *      the sum over its rows [r M/k, (r+1) M/k) of the sequence;
 *  12. the block's residual connection x + mlp(x) (the TransformerBlock of
 *      §3.4 on the page above) is added to that block:
 *      O_r = X[rows of r] + Z[rows of r].
 *
 * SwiGLU variant of the block (gate_proj and up_proj column-parallel,
 * down_proj row-parallel: §6.1 of the page above; gate_up_proj column- and
 * down_proj row-parallel for Llama-2-70B: "大模型分布式优化技术（一）"
 * §5.1, which names the SwiGLU activation in §3.3); the formula is not on
 * the pages and is taken as Llama's, without biases:
 *  13. Y_i = SiLU(X Wg_i) * (X Wu_i), SiLU(x) = x sigma(x) = x / (1 + e^-x),
 *      with Wg_i, Wu_i the column blocks i of Wg, Wu [H, F]; steps 4 and 5
 *      are unchanged (Z_i = Y_i V_i, Z = sum_i Z_i).
 *
 * Tensor-parallel attention block (multi-head attention split by heads: the
 * Q/K/V projections column-parallel, each shard computing its own heads'
 * attention with no communication, the output projection row-parallel and
 * summed: "AI大模型分布式训练：张量并行与流水线并行深度实践" §2.3; "千亿参数模型如何拆分
 * 到多张GPU上训练" 注意力层的切分; "大模型分布式并行策略详解：TP、DP、PP、CP、EP核心原理
 * 与实战" §4.2).  Given Wq, Wk, Wv, Wo [H, H], biases bq, bk, bv [H], n_heads
 * heads of d = H / n_heads columns, k shards of hk = n_heads / k heads and
 * Hk = hk d, rows m = b S + t of X (batch b, position t):
 *  14. shard i's heads are i hk .. (i+1) hk - 1; its projection output is
 *      [q | k | v] = X [Wq_i | Wk_i | Wv_i] + [bq_i | bk_i | bv_i] with
 *      Wq_i = Wq[:, i Hk:(i+1) Hk] (and so on), the chunk-in-three layout of
 *      the shard's ColumnParallelLinear(H, 3H) output;
 *  15. per head h, scaled dot-product attention within each sequence:
 *      s_tj = q_t . k_j / sqrt(d) for keys j of the same sequence, j <= t
 *      when causal; p_tj = exp(s_tj) / sum_j' exp(s_tj'); o_t = sum_j p_tj v_j;
 *  16. A_i = the shard's heads side by side [M, Hk]; Z_i = A_i Wo_i with
 *      Wo_i = Wo[i Hk:(i+1) Hk, :] (RowParallelLinear, no bias);
 *  17. Z = Z_0 + ... + Z_{k-1}.
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

/* ---------------------------------------------------------------------- */
/* Backward.                                                               */

/* GeLU'(x) = Phi(x) + x phi(x) (step 8), Phi as in oracle_gelu. */
double oracle_gelu_grad(double x) {
  const double inv_sqrt_2pi = 0.39894228040143267793994605993438;
  return 0.5 * erfc(-x / sqrt(2.0)) + x * exp(-0.5 * x * x) * inv_sqrt_2pi;
}

void oracle_gelu_grad_array(const double* x, int64_t n, double* g) {
  for (int64_t i = 0; i < n; ++i) g[i] = oracle_gelu_grad(x[i]);
}

/* G_i[M,Fk] = GeLU'(X W_i + b_i) of shard i (steps 2 and 8). */
void oracle_col_gelu_grad(const double* X, const double* W, const double* b, int64_t M, int64_t H,
                          int64_t F, int k, int i, double* G) {
  const int64_t Fk = F / k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) {
    double* g = G + m * Fk;
    preact_row(X, W, b, m, H, F, Fk, i, g);
    for (int64_t j = 0; j < Fk; ++j) g[j] = oracle_gelu_grad(g[j]);
  }
}

/* One row of steps 7-8: da[j] = g[j] * sum_n dz[n] V[i*Fk + j, n]. */
static void act_grad_row(const double* dz, const double* V, const double* g, int64_t H, int64_t Fk,
                         int64_t i, double* da) {
  for (int64_t j = 0; j < Fk; ++j) {
    const double* v = V + (i * Fk + j) * H;
    double s = 0.0;
    for (int64_t n = 0; n < H; ++n) s += dz[n] * v[n];
    da[j] = s * g[j];
  }
}

/* dA_i[M,Fk] = (dZ V_i^T) * G_i (steps 7-8); V is the full [F,H] matrix. */
void oracle_act_grad(const double* dZ, const double* V, const double* Gi, int64_t M, int64_t F,
                     int64_t H, int k, int i, double* dAi) {
  const int64_t Fk = F / k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) act_grad_row(dZ + m * H, V, Gi + m * Fk, H, Fk, i, dAi + m * Fk);
}

/* dV_i[Fk,H]: dV_i[j,n] = sum_m Y_i[m,j] dZ[m,n] (step 7). */
void oracle_row_weight_grad(const double* Yi, const double* dZ, int64_t M, int64_t Fk, int64_t H,
                            double* dVi) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < Fk; ++j) {
    double* out = dVi + j * H;
    for (int64_t n = 0; n < H; ++n) out[n] = 0.0;
    for (int64_t m = 0; m < M; ++m) {
      const double y = Yi[m * Fk + j];
      const double* dz = dZ + m * H;
      for (int64_t n = 0; n < H; ++n) out[n] += y * dz[n];
    }
  }
}

/* dW_i[H,Fk]: dW_i[h,j] = sum_m X[m,h] dA_i[m,j], and db_i[j] = sum_m dA_i[m,j]
   (step 9).  db_i may be NULL. */
void oracle_col_weight_grad(const double* X, const double* dAi, int64_t M, int64_t H, int64_t Fk,
                            double* dWi, double* dbi) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t h = 0; h < H; ++h) {
    double* out = dWi + h * Fk;
    for (int64_t j = 0; j < Fk; ++j) out[j] = 0.0;
    for (int64_t m = 0; m < M; ++m) {
      const double x = X[m * H + h];
      const double* da = dAi + m * Fk;
      for (int64_t j = 0; j < Fk; ++j) out[j] += x * da[j];
    }
  }
  if (dbi) {
    for (int64_t j = 0; j < Fk; ++j) dbi[j] = 0.0;
    for (int64_t m = 0; m < M; ++m)
      for (int64_t j = 0; j < Fk; ++j) dbi[j] += dAi[m * Fk + j];
  }
}

/* One row of step 9's input gradient: dx[h] = sum_j da[j] W[h, i*Fk + j]. */
static void input_grad_row(const double* da, const double* W, int64_t H, int64_t F, int64_t Fk,
                           int64_t i, double* dx) {
  for (int64_t h = 0; h < H; ++h) {
    const double* w = W + h * F + i * Fk;
    double s = 0.0;
    for (int64_t j = 0; j < Fk; ++j) s += da[j] * w[j];
    dx[h] = s;
  }
}

/* dX_i[M,H] = dA_i W_i^T (step 9); W is the full [H,F] matrix. */
void oracle_input_grad_partial(const double* dAi, const double* W, int64_t M, int64_t H, int64_t F,
                               int k, int i, double* dXi) {
  const int64_t Fk = F / k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) input_grad_row(dAi + m * Fk, W, H, F, Fk, i, dXi + m * H);
}

/* Whole backward for selected rows of dX (steps 6-10 for each row, which
   only needs that row of X and dZ): dX[r,:] = sum_i dA_i[m,:] W_i^T with
   m = rows[r] (rows == NULL: 0..nrows-1).  b may be NULL. */
void oracle_backward_rows(const double* X, const double* W, const double* b, const double* V,
                          const double* dZ, int64_t H, int64_t F, int k, const int64_t* rows,
                          int64_t nrows, double* dX) {
  const int64_t Fk = F / k;
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)Fk);
    double* da = (double*)malloc(sizeof(double) * (size_t)Fk);
    double* dxi = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t m = rows ? rows[r] : r;
      double* dx = dX + r * H;
      for (int64_t h = 0; h < H; ++h) dx[h] = 0.0;
      for (int i = 0; i < k; ++i) {
        preact_row(X, W, b, m, H, F, Fk, i, g);                        /* step 2 */
        for (int64_t j = 0; j < Fk; ++j) g[j] = oracle_gelu_grad(g[j]); /* step 8 */
        act_grad_row(dZ + m * H, V, g, H, Fk, i, da);                   /* steps 7-8 */
        input_grad_row(da, W, H, F, Fk, i, dxi);                        /* step 9 */
        for (int64_t h = 0; h < H; ++h) dx[h] += dxi[h];                /* step 10 */
      }
    }
    free(g);
    free(da);
    free(dxi);
  }
}

/* Parameter gradients for selected columns c of the full F (shard c / Fk):
   dWc[r,:] = dW[:, c] (H values), dbc[r] = db[c], dVc[r,:] = dV[c, :], with
   c = cols[r].  Column c of A = X W + b, and so of Y, G and dA, depends on
   column c of W, entry c of b and row c of V only. */
void oracle_backward_cols(const double* X, const double* W, const double* b, const double* V,
                          const double* dZ, int64_t M, int64_t H, int64_t F, const int64_t* cols,
                          int64_t ncols, double* dWc, double* dbc, double* dVc) {
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    double* da = (double*)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(H > 0 ? H : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < ncols; ++r) {
      const int64_t c = cols[r];
      const double* v = V + c * H;
      for (int64_t h = 0; h < H; ++h) w[h] = W[h * F + c];              /* column c of W */
      for (int64_t m = 0; m < M; ++m) {
        const double* x = X + m * H;
        const double* dz = dZ + m * H;
        double a = 0.0;                                                  /* step 2 */
        for (int64_t h = 0; h < H; ++h) a += x[h] * w[h];
        if (b) a += b[c];
        double s = 0.0;                                                  /* step 7 */
        for (int64_t n = 0; n < H; ++n) s += dz[n] * v[n];
        y[m] = oracle_gelu(a);                                           /* step 3 */
        da[m] = s * oracle_gelu_grad(a);                                 /* step 8 */
      }
      /* dW[:, c] = X^T da, db[c] = sum da (step 9) and dV[c, :] = y^T dZ
         (step 7): every sum runs over m = 0 .. M-1 in order, one row of X
         and of dZ at a time. */
      double* dw = dWc + r * H;
      double* dv = dVc + r * H;
      for (int64_t h = 0; h < H; ++h) dw[h] = 0.0;
      for (int64_t n = 0; n < H; ++n) dv[n] = 0.0;
      double sb = 0.0;
      for (int64_t m = 0; m < M; ++m) {
        const double* x = X + m * H;
        const double* dz = dZ + m * H;
        const double d = da[m], ym = y[m];
        for (int64_t h = 0; h < H; ++h) dw[h] += x[h] * d;
        for (int64_t n = 0; n < H; ++n) dv[n] += ym * dz[n];
        sb += d;
      }
      dbc[r] = sb;
    }
    free(y);
    free(da);
    free(w);
  }
}

/* ---------------------------------------------------------------------- */
/* Sequence parallelism (steps 11-12).                                     */

/* For each rank r < k, rows [r*Mb, (r+1)*Mb) with Mb = M / k (k divides M):
   out[r][m*H + n] = R[(r*Mb + m)*H + n] + sum_i parts[i][(r*Mb + m)*H + n],
   the sum over parts in index order.  R == NULL: no residual. */
void oracle_sp_reduce_scatter(const double* const* parts, int nparts, const double* R, int k,
                              int64_t M, int64_t H, double* const* out) {
  const int64_t Mb = M / k;
  for (int r = 0; r < k; ++r) {
    double* o = out[r];
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < Mb; ++m) {
      const int64_t row = r * Mb + m;
      for (int64_t n = 0; n < H; ++n) {
        double s = 0.0;
        for (int i = 0; i < nparts; ++i) s += parts[i][row * H + n];
        o[m * H + n] = (R ? R[row * H + n] : 0.0) + s;
      }
    }
  }
}

/* ---------------------------------------------------------------------- */
/* SwiGLU (step 13).                                                       */

/* SiLU(x) = x sigma(x) = x / (1 + exp(-x)); for x -> -inf, exp(-x)
   overflows to +inf and the quotient is (-)0, the limit. */
double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

void oracle_silu_array(const double* x, int64_t n, double* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = oracle_silu(x[i]);
}

/* Y_i[M,Fk] = SiLU(X Wg_i) * (X Wu_i) of shard i. */
void oracle_swiglu_col(const double* X, const double* Wg, const double* Wu, int64_t M, int64_t H,
                       int64_t F, int k, int i, double* Y) {
  const int64_t Fk = F / k;
#pragma omp parallel
  {
    double* u = (double*)malloc(sizeof(double) * (size_t)(Fk > 0 ? Fk : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
      double* y = Y + m * Fk;
      preact_row(X, Wg, NULL, m, H, F, Fk, i, y);
      preact_row(X, Wu, NULL, m, H, F, Fk, i, u);
      for (int64_t j = 0; j < Fk; ++j) y[j] = oracle_silu(y[j]) * u[j];
    }
    free(u);
  }
}

/* Whole SwiGLU forward for selected rows (steps 13, 4, 5):
   Z[r, :] = sum_i (SiLU(x Wg_i) * (x Wu_i)) V_i with x = X[rows[r], :]
   (rows == NULL: 0..nrows-1). */
void oracle_swiglu_forward_rows(const double* X, const double* Wg, const double* Wu,
                                const double* V, int64_t H, int64_t F, int k, const int64_t* rows,
                                int64_t nrows, double* Z) {
  const int64_t Fk = F / k;
#pragma omp parallel
  {
    double* y = (double*)malloc(sizeof(double) * (size_t)Fk);
    double* u = (double*)malloc(sizeof(double) * (size_t)Fk);
    double* zi = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t m = rows ? rows[r] : r;
      double* z = Z + r * H;
      for (int64_t n = 0; n < H; ++n) z[n] = 0.0;
      for (int i = 0; i < k; ++i) {
        preact_row(X, Wg, NULL, m, H, F, Fk, i, y);
        preact_row(X, Wu, NULL, m, H, F, Fk, i, u);
        for (int64_t j = 0; j < Fk; ++j) y[j] = oracle_silu(y[j]) * u[j];
        partial_row(y, V, H, Fk, i, zi);
        for (int64_t n = 0; n < H; ++n) z[n] += zi[n];
      }
    }
    free(y);
    free(u);
    free(zi);
  }
}

/* ---------------------------------------------------------------------- */
/* Tensor-parallel attention (steps 14-17).                                 */

/* Step 14 for one row: out[0..3Hk) = [q | k | v] of shard i. */
static void attn_qkv_row(const double* x, const double* Wq, const double* Wk, const double* Wv,
                         const double* bq, const double* bk, const double* bv, int64_t H,
                         int64_t Hk, int64_t i, double* out) {
  const double* W[3] = {Wq, Wk, Wv};
  const double* bb[3] = {bq, bk, bv};
  for (int part = 0; part < 3; ++part) {
    double* o = out + part * Hk;
    for (int64_t c = 0; c < Hk; ++c) o[c] = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      const double xv = x[h];
      const double* w = W[part] + h * H + i * Hk;
      for (int64_t c = 0; c < Hk; ++c) o[c] += xv * w[c];
    }
    if (bb[part])
      for (int64_t c = 0; c < Hk; ++c) o[c] += bb[part][i * Hk + c];
  }
}

/* QKV_i[M, 3 Hk] of shard i (step 14).  Biases may be NULL. */
void oracle_attn_qkv(const double* X, const double* Wq, const double* Wk, const double* Wv,
                     const double* bq, const double* bk, const double* bv, int64_t M, int64_t H,
                     int nh, int k, int i, double* QKV) {
  const int64_t Hk = H / nh * (nh / k);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < M; ++m) attn_qkv_row(X + m * H, Wq, Wk, Wv, bq, bk, bv, H, Hk, i, QKV + m * 3 * Hk);
}

/* Step 15 for one query row t of sequence b and one head h of the shard:
   qkv is the shard's [M, 3 Hk] projection, o[0..d) the head's output. */
static void attn_head_row(const double* qkv, int64_t S, int64_t Hk, int64_t d, int64_t b, int64_t t,
                          int64_t h, int causal, double* p, double* o) {
  const int64_t ld = 3 * Hk;
  const double* q = qkv + (b * S + t) * ld + h * d;
  const int64_t nkeys = causal ? t + 1 : S;
  const double scale = 1.0 / sqrt((double)d);
  double mx = -INFINITY;
  for (int64_t j = 0; j < nkeys; ++j) {
    const double* kj = qkv + (b * S + j) * ld + Hk + h * d;
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += q[c] * kj[c];
    p[j] = s * scale;
    if (p[j] > mx) mx = p[j];
  }
  /* softmax; subtracting the maximum changes no value in exact arithmetic */
  double sum = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    p[j] = exp(p[j] - mx);
    sum += p[j];
  }
  for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
  for (int64_t j = 0; j < nkeys; ++j) {
    const double w = p[j] / sum;
    const double* vj = qkv + (b * S + j) * ld + 2 * Hk + h * d;
    for (int64_t c = 0; c < d; ++c) o[c] += w * vj[c];
  }
}

/* A_i[M, Hk] from the shard's projection QKV_i (step 15), M = B S. */
void oracle_attn_core(const double* QKV, int64_t B, int64_t S, int hk, int64_t d, int causal,
                      double* A) {
  const int64_t Hk = hk * d;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < S; ++t)
        for (int64_t h = 0; h < hk; ++h) attn_head_row(QKV, S, Hk, d, b, t, h, causal, p, A + (b * S + t) * Hk + h * d);
    free(p);
  }
}

/* Selected rows of A_i (step 15): A[r, :] for row m = rows[r] = b S + t of
   the shard's projection QKV_i [B S, 3 Hk], every head of the shard; the
   same per-row evaluation as oracle_attn_core. */
void oracle_attn_core_rows(const double* QKV, int64_t S, int hk, int64_t d, int causal,
                           const int64_t* rows, int64_t nrows, double* A) {
  const int64_t Hk = hk * d;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t r = 0; r < nrows; ++r)
      for (int64_t h = 0; h < hk; ++h)
        attn_head_row(QKV, S, Hk, d, rows[r] / S, rows[r] % S, h, causal, p, A + r * Hk + h * d);
    free(p);
  }
}

/* The whole block for selected rows (steps 14-17): Z[r, :] for row
   m = rows[r] = b S + t.  Only the rows the query attends to are projected
   (positions 0..t of sequence b when causal, the whole sequence otherwise). */
void oracle_attn_forward_rows(const double* X, const double* Wq, const double* Wk, const double* Wv,
                              const double* bq, const double* bk, const double* bv, const double* Wo,
                              int64_t S, int64_t H, int nh, int k, int causal, const int64_t* rows,
                              int64_t nrows, double* Z) {
  const int64_t d = H / nh, hk = nh / k, Hk = hk * d;
#pragma omp parallel
  {
    double* qkv = (double*)malloc(sizeof(double) * (size_t)(S * 3 * Hk));
    double* p = (double*)malloc(sizeof(double) * (size_t)S);
    double* a = (double*)malloc(sizeof(double) * (size_t)Hk);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      const int64_t m = rows[r], b = m / S, t = m % S;
      const int64_t n = causal ? t + 1 : S;
      double* z = Z + r * H;
      for (int64_t c = 0; c < H; ++c) z[c] = 0.0;
      for (int i = 0; i < k; ++i) {
        /* the shard's projection of rows b S .. b S + n - 1, stored as a
           one-sequence [n, 3 Hk] block (sequence 0 of length n) */
        for (int64_t j = 0; j < n; ++j)
          attn_qkv_row(X + (b * S + j) * H, Wq, Wk, Wv, bq, bk, bv, H, Hk, i, qkv + j * 3 * Hk);
        for (int64_t h = 0; h < hk; ++h)
          attn_head_row(qkv, n, Hk, d, 0, t, h, causal, p, a + h * d);
        /* Z += A_i[m] Wo_i */
        for (int64_t c = 0; c < Hk; ++c) {
          const double av = a[c];
          const double* w = Wo + (i * Hk + c) * H;
          for (int64_t e = 0; e < H; ++e) z[e] += av * w[e];
        }
      }
    }
    free(qkv);
    free(p);
    free(a);
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

/* SHA-256 of this file's text, passed on the compiler command line by the
   build, so that the loader can refuse a library built from an older copy
   of the source instead of running stale arithmetic. */
#ifndef ORACLE_SOURCE_SHA256
#define ORACLE_SOURCE_SHA256 "unknown"
#endif
const char* oracle_source_sha256(void) { return ORACLE_SOURCE_SHA256; }
