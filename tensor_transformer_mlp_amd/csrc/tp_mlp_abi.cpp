// C ABI of libtpmlp.so (declared in include/tp_mlp.h): argument checks, the
// shard loops and the workspace layouts.  Every check runs on the host before
// the first HIP call, so a rejected call launches nothing.
#include "tp_mlp.h"
#include "tp_mlp_dev.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_mlp_kernels.h"

namespace {

using tpmlp::GemmArgs;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxLd = int64_t(1) << 22;  // H, Fk: 32-bit row offsets inside a tile
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elt_size(int dtype) { return dtype == TP_BF16 ? 2 : 4; }

// Shape rules shared by every entry point.  M may be 0.
int check_dims(int64_t M, int64_t H, int64_t Fk) {
  if (M < 0 || M > kMaxDim) return TP_ERR_SHAPE;
  if (H < 8 || H > kMaxLd || H % 8) return TP_ERR_SHAPE;
  if (Fk < 8 || Fk > kMaxLd || Fk % 8) return TP_ERR_SHAPE;
  if (M > 0 && (M > kMaxElems / H || M > kMaxElems / Fk)) return TP_ERR_SHAPE;
  if (H > kMaxElems / Fk) return TP_ERR_SHAPE;
  return TP_OK;
}

int check_dtype(int dtype) { return (dtype == TP_F32 || dtype == TP_BF16) ? TP_OK : TP_ERR_DTYPE; }

// [a, a + na) and [b, b + nb) overlap (bytes)?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

// A set of byte ranges: outputs may overlap neither an input nor each other.
struct Region {
  const void* p;
  size_t n;
};
struct Regions {
  static constexpr int kMax = 4 * TP_MAX_SHARDS + 8;
  Region r[kMax];
  int n = 0;
  void add(const void* p, size_t bytes) {
    if (p && bytes && n < kMax) r[n++] = Region{p, bytes};
  }
};
bool any_overlap(const Regions& outs, const Regions& ins) {
  for (int i = 0; i < outs.n; ++i) {
    for (int j = 0; j < ins.n; ++j)
      if (overlap(outs.r[i].p, outs.r[i].n, ins.r[j].p, ins.r[j].n)) return true;
    for (int j = 0; j < i; ++j)
      if (overlap(outs.r[i].p, outs.r[i].n, outs.r[j].p, outs.r[j].n)) return true;
  }
  return false;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

using tpmlp::GemmBatch;
using tpmlp::kMaxGroups;

// The shards of a step are launched together in batches of up to kMaxGroups.
int batch_size(int k) { return k < kMaxGroups ? k : kMaxGroups; }

GemmBatch batch(int n, tpmlp::Layout layout, tpmlp::Epilogue epi, int64_t M, int64_t N, int64_t K,
                int64_t lda, int64_t ldb) {
  GemmBatch b{};
  b.groups = n;
  b.group_sum = false;
  b.M = M;
  b.N = N;
  b.K = K;
  b.lda = lda;
  b.ldb = ldb;
  b.ldc = N;
  b.layout = layout;
  b.epi = epi;
  return b;
}

// tile >= 0 (bf16 only, checked by the caller): that tile of the GEMM's table
// instead of the one the library picks.
int run(const GemmBatch& b, int dtype, hipStream_t s, int tile = -1) {
  if (tile >= 0) return hip_status(tpmlp::launch_gemm_bf16_batch_tile(tile, b, s));
  return hip_status(dtype == TP_BF16 ? tpmlp::launch_gemm_bf16_batch(b, s)
                                     : tpmlp::launch_gemm_f32_batch(b, s));
}

// The steps, after validation; arrays hold the n shards of one batch.
// Y_i (and G_i) = act(X W_i + b_i): [M, H] x [H, Fk], both row-major.
GemmBatch col_batch(const void* X, const void* const* W, const void* const* b, void* const* Y,
                    void* const* G, int n, int64_t M, int64_t H, int64_t Fk) {
  GemmBatch g = batch(n, tpmlp::kNN, G ? tpmlp::kEpiBiasGeluSave : tpmlp::kEpiBiasGelu, M, Fk, H, H, Fk);
  for (int i = 0; i < n; ++i) {
    g.A[i] = X;
    g.B[i] = W ? W[i] : nullptr;
    g.bias[i] = b ? b[i] : nullptr;
    g.C[i] = Y ? Y[i] : nullptr;
    g.aux[i] = G ? G[i] : nullptr;
  }
  return g;
}

int col_steps(const void* X, const void* const* W, const void* const* b, void* const* Y,
              void* const* G, int n, int64_t M, int64_t H, int64_t Fk, int dtype, hipStream_t s,
              int tile = -1) {
  return run(col_batch(X, W, b, Y, G, n, M, H, Fk), dtype, s, tile);
}

// SwiGLU column step: Y_i = SiLU(X Wg_i) * (X Wu_i), two [H, Fk] row-major
// weights per shard in one GEMM.
int swiglu_col_steps(const void* X, const void* const* Wg, const void* const* Wu, void* const* Y, int n,
                     int64_t M, int64_t H, int64_t Fk, int dtype, hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kNN, tpmlp::kEpiSwiGLU, M, Fk, H, H, Fk);
  for (int i = 0; i < n; ++i) {
    g.A[i] = X;
    g.B[i] = Wg[i];
    g.B2[i] = Wu[i];
    g.C[i] = Y[i];
  }
  return run(g, dtype, s);
}

// Attention projection: QKV_i = X Wqkv_i + bqkv_i, [M, H] x [H, 3 Hk].
int qkv_steps(const void* X, const void* const* W, const void* const* b, void* const* QKV, int n, int64_t M,
              int64_t H, int64_t Hk, int dtype, hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kNN, tpmlp::kEpiBias, M, 3 * Hk, H, H, 3 * Hk);
  for (int i = 0; i < n; ++i) {
    g.A[i] = X;
    g.B[i] = W[i];
    g.bias[i] = b ? b[i] : nullptr;
    g.C[i] = QKV[i];
  }
  return run(g, dtype, s);
}

// Shape rules of the attention block: d = H / n_heads in {64, 128}, k | n_heads,
// and one sequence's projection rows addressable with 32-bit offsets.
int check_attn(int64_t B, int64_t S, int64_t H, int n_heads, int k) {
  if (B < 0 || S < 0 || B > kMaxDim || S > kMaxDim) return TP_ERR_SHAPE;
  if (n_heads < 1 || k < 1 || k > TP_MAX_SHARDS || H % 8 || H < 8 || H > kMaxLd) return TP_ERR_SHAPE;
  if (H % n_heads || n_heads % k) return TP_ERR_SHAPE;
  const int64_t d = H / n_heads;
  if (d != 64 && d != 128) return TP_ERR_SHAPE;
  const int64_t Hk = d * (n_heads / k);
  if (S > 0 && S > ((int64_t(1) << 31) - 1) / (6 * Hk)) return TP_ERR_SHAPE;
  if (B > 0 && S > 0 && B > kMaxDim / S) return TP_ERR_SHAPE;
  return check_dims(B * S, H, Hk);
}

// Z_i (+)= Y_i V_i: [M, Fk] x [Fk, H], one output per shard (sum == false),
// or Z (+)= sum_i Y_i V_i in shard order into Z[0] (sum == true).
GemmBatch row_batch(const void* const* Y, const void* const* V, float* const* Z, int n, bool sum,
                    int64_t M, int64_t Fk, int64_t H, bool accumulate) {
  GemmBatch g = batch(n, tpmlp::kNN, accumulate ? tpmlp::kEpiAccumF32 : tpmlp::kEpiStoreF32, M, H, Fk,
                      Fk, H);
  g.group_sum = sum;
  for (int i = 0; i < n; ++i) {
    g.A[i] = Y ? Y[i] : nullptr;
    g.B[i] = V ? V[i] : nullptr;
    g.C[i] = Z ? (sum ? Z[0] : Z[i]) : nullptr;
  }
  return g;
}

int row_steps(const void* const* Y, const void* const* V, float* const* Z, int n, bool sum,
              int64_t M, int64_t Fk, int64_t H, int dtype, bool accumulate, hipStream_t s,
              int tile = -1) {
  return run(row_batch(Y, V, Z, n, sum, M, Fk, H, accumulate), dtype, s, tile);
}

// dA_i = (dZ V_i^T) * G_i: [M, H] x ([Fk, H] read as its transpose).
int act_grad_steps(const void* dZ, const void* const* V, const void* const* G, void* const* dA, int n,
                   int64_t M, int64_t H, int64_t Fk, int dtype, hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kNT, tpmlp::kEpiMulAux, M, Fk, H, H, H);
  for (int i = 0; i < n; ++i) {
    g.A[i] = dZ;
    g.B[i] = V[i];
    g.C[i] = dA[i];
    g.aux[i] = const_cast<void*>(G[i]);
  }
  return run(g, dtype, s);
}

// Weight-gradient workspace for a batch of `groups` shards: the larger
// K-split of the two weight GEMMs, then the column-sum partials of the batch.
size_t split_bytes(int groups, int64_t M, int64_t H, int64_t Fk, int dtype) {
  const bool bf16 = dtype == TP_BF16;
  const size_t a = tpmlp::gemm_split_workspace_bytes(bf16, groups, Fk, H, M);
  const size_t b = tpmlp::gemm_split_workspace_bytes(bf16, groups, H, Fk, M);
  return round_up(a > b ? a : b, kWsAlign);
}
size_t colsum_bytes(int groups, int64_t M, int64_t Fk) {
  return round_up(size_t(groups) * size_t(tpmlp::colsum_partials_floats(M, Fk)) * 4, kWsAlign);
}
size_t grad_weight_ws(int groups, int64_t M, int64_t H, int64_t Fk, int dtype) {
  return split_bytes(groups, M, H, Fk, dtype) + colsum_bytes(groups, M, Fk);
}

// The whole backward multiplies by V_i^T and W_i^T through transposed copies
// of the weights (N-major operands: the GEMM's NN path, which on the same
// shapes runs 8-32% faster than the NT path reading them as transposes) when
// the token count makes the products outweigh the copies: bf16 and M >= 4096.
// Measured on the whole backward, bit-identical: 3.8% faster on gpt2_small's
// shards, 2.6% on long_seq's, 0.5% on llama7b's; gpt3_175b's (M = 2048, 151 MB
// weights per shard) keep the NT path.
constexpr int64_t kTransposeMinRows = 4096;
bool backward_transposes(int64_t M, int dtype) { return dtype == TP_BF16 && M >= kTransposeMinRows; }

// dV_i (+)= Y_i^T dZ: ([M, Fk] read as its transpose) x [M, H], K = M.
int row_weight_steps(const void* const* Y, const void* dZ, float* const* dV, int n, int64_t M,
                     int64_t Fk, int64_t H, int dtype, void* ws, bool accumulate, hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kTN, accumulate ? tpmlp::kEpiAccumF32 : tpmlp::kEpiStoreF32, Fk, H, M,
                      Fk, H);
  for (int i = 0; i < n; ++i) {
    g.A[i] = Y[i];
    g.B[i] = dZ;
    g.C[i] = dV[i];
  }
  return hip_status(tpmlp::launch_gemm_split(g, dtype == TP_BF16, ws, s));
}

// dW_i (+)= X^T dA_i and db_i (+)= colsum(dA_i).
int col_weight_steps(const void* X, const void* const* dA, float* const* dW, float* const* db, int n,
                     int64_t M, int64_t H, int64_t Fk, int dtype, void* ws, bool accumulate,
                     hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kTN, accumulate ? tpmlp::kEpiAccumF32 : tpmlp::kEpiStoreF32, H, Fk, M,
                      H, Fk);
  for (int i = 0; i < n; ++i) {
    g.A[i] = X;
    g.B[i] = dA[i];
    g.C[i] = dW[i];
  }
  int st = hip_status(tpmlp::launch_gemm_split(g, dtype == TP_BF16, ws, s));
  if (st || !db) return st;
  float* partials =
      reinterpret_cast<float*>(static_cast<char*>(ws) + split_bytes(n, M, H, Fk, dtype));
  return hip_status(
      tpmlp::launch_colsum(dA, n, dtype == TP_BF16, M, Fk, db, accumulate, partials, s));
}

// dX_i (+)= dA_i W_i^T: [M, Fk] x ([H, Fk] read as its transpose); one output
// per shard, or the shard-order sum into dX[0] (sum == true).
// dA_i = (dZ Vt_i) * G_i with Vt_i = V_i^T stored [H, Fk] (N-major: the NN
// path of the GEMM; the same products as act_grad_steps).
int act_grad_nn_steps(const void* dZ, void* const* Vt, const void* const* G, void* const* dA, int n,
                      int64_t M, int64_t H, int64_t Fk, int dtype, hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kNN, tpmlp::kEpiMulAux, M, Fk, H, H, Fk);
  for (int i = 0; i < n; ++i) {
    g.A[i] = dZ;
    g.B[i] = Vt[i];
    g.C[i] = dA[i];
    g.aux[i] = const_cast<void*>(G[i]);
  }
  return run(g, dtype, s);
}

int input_grad_steps(const void* const* dA, const void* const* W, float* const* dX, int n, bool sum,
                     int64_t M, int64_t Fk, int64_t H, int dtype, bool accumulate, hipStream_t s) {
  GemmBatch g = batch(n, tpmlp::kNT, accumulate ? tpmlp::kEpiAccumF32 : tpmlp::kEpiStoreF32, M, H, Fk,
                      Fk, Fk);
  g.group_sum = sum;
  for (int i = 0; i < n; ++i) {
    g.A[i] = dA[i];
    g.B[i] = W[i];
    g.C[i] = sum ? dX[0] : dX[i];
  }
  return run(g, dtype, s);
}

// The column and row steps of k shards, in batches of up to G (<= kMaxGroups)
// shards per launch.  col(i0, n) runs the column step of shards i0 ..
// i0 + n - 1 into Y[0 .. n-1].  Literal (fused == false): partial i goes to
// part(i) and its pointer to parts[i].  Fused: the row step of every batch
// adds its shards, in shard order, into part(0) (the first batch stores).
// The batch size changes no result bit.
template <class Col, class Part>
int shard_steps(Col col, const void* const* V, int k, int64_t M, int64_t H, int64_t Fk, int dtype,
                void* const* Y, bool fused, Part part, const float** parts, hipStream_t s, int G) {
  float* P[kMaxGroups];
  int st;
  for (int i0 = 0; i0 < k; i0 += G) {
    const int n = k - i0 < G ? k - i0 : G;
    if ((st = col(i0, n))) return st;
    if (fused) {
      P[0] = part(0);
      if ((st = row_steps(Y, V + i0, P, n, true, M, Fk, H, dtype, i0 > 0, s))) return st;
    } else {
      for (int j = 0; j < n; ++j) {
        P[j] = part(i0 + j);
        parts[i0 + j] = P[j];
      }
      if ((st = row_steps(Y, V + i0, P, n, false, M, Fk, H, dtype, false, s))) return st;
    }
  }
  return TP_OK;
}

// Shape and pointer rules of the sequence-parallel reduce-scatter.
int check_sp(const float* const* parts, int nparts, const void* R, int r_dtype, void* const* O,
             int out_dtype, int k, int64_t M, int64_t H) {
  if (check_dtype(r_dtype) || check_dtype(out_dtype)) return TP_ERR_DTYPE;
  if (nparts < 1 || nparts > TP_MAX_SHARDS || k < 1 || k > TP_MAX_SHARDS) return TP_ERR_SHAPE;
  if (check_dims(M, H, 8)) return TP_ERR_SHAPE;
  if (M % k) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (!parts || !O) return TP_ERR_NULL;
  for (int i = 0; i < nparts; ++i) {
    if (!parts[i]) return TP_ERR_NULL;
    if (!aligned16(parts[i])) return TP_ERR_ALIGN;
  }
  for (int r = 0; r < k; ++r) {
    if (!O[r]) return TP_ERR_NULL;
    if (!aligned16(O[r])) return TP_ERR_ALIGN;
  }
  if (R && !aligned16(R)) return TP_ERR_ALIGN;
  const size_t nz = size_t(M) * size_t(H);
  Regions in, out;
  for (int i = 0; i < nparts; ++i) in.add(parts[i], nz * 4);
  if (R) in.add(R, nz * elt_size(r_dtype));
  for (int r = 0; r < k; ++r) out.add(O[r], nz / size_t(k) * elt_size(out_dtype));
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return TP_OK;
}

// tp_mlp_col_gelu_shards after the tile argument's own checks (tile < 0: the
// library's choice).
int col_shards(const void* X, const void* const* W, const void* const* b, void* const* Y,
               void* const* G, int n, int64_t M, int64_t H, int64_t Fk, int dtype, void* stream,
               int tile) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (!X || !W || !Y) return TP_ERR_NULL;
  if (!aligned16(X)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * e);
  for (int i = 0; i < n; ++i) {
    if (!W[i] || !Y[i] || (b && !b[i]) || (G && !G[i])) return TP_ERR_NULL;
    if (!aligned16(W[i]) || !aligned16(Y[i]) || (b && !aligned16(b[i])) || (G && !aligned16(G[i])))
      return TP_ERR_ALIGN;
    in.add(W[i], size_t(H) * size_t(Fk) * e);
    if (b) in.add(b[i], size_t(Fk) * e);
    out.add(Y[i], size_t(M) * size_t(Fk) * e);
    if (G) out.add(G[i], size_t(M) * size_t(Fk) * e);
  }
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return col_steps(X, W, b, Y, G, n, M, H, Fk, dtype, static_cast<hipStream_t>(stream), tile);
}

// tp_mlp_row_partial_shards after the tile argument's own checks (tile < 0:
// the library's choice).
int row_shards(const void* const* Y, const void* const* V, float* const* Z, int n, int64_t M,
               int64_t Fk, int64_t H, int dtype, unsigned flags, void* stream, int tile) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~(TP_ACCUMULATE | TP_SUM_SHARDS)) return TP_ERR_FLAGS;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  const bool sum = (flags & TP_SUM_SHARDS) != 0;
  if (!Y || !V || !Z) return TP_ERR_NULL;
  const size_t e = elt_size(dtype);
  Regions in, out;
  for (int i = 0; i < n; ++i) {
    if (!Y[i] || !V[i] || ((!sum || i == 0) && !Z[i])) return TP_ERR_NULL;
    if (!aligned16(Y[i]) || !aligned16(V[i]) || ((!sum || i == 0) && !aligned16(Z[i])))
      return TP_ERR_ALIGN;
    in.add(Y[i], size_t(M) * size_t(Fk) * e);
    in.add(V[i], size_t(Fk) * size_t(H) * e);
    if (!sum || i == 0) out.add(Z[i], size_t(M) * size_t(H) * 4);
  }
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return row_steps(Y, V, Z, n, sum, M, Fk, H, dtype, (flags & TP_ACCUMULATE) != 0,
                   static_cast<hipStream_t>(stream), tile);
}

// Argument rules of the whole forward (everything but the workspace).
int check_forward(const void* X, const void* const* W, const void* const* b, const void* const* V, int k,
                  int64_t M, int64_t H, int64_t Fk, int dtype, const float* Z, unsigned flags) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~TP_FUSED_ACCUM) return TP_ERR_FLAGS;
  if (k < 1 || k > TP_MAX_SHARDS) return TP_ERR_SHAPE;
  if ((st = check_dims(M, H, Fk))) return st;
  if (M == 0) return TP_OK;
  if (!X || !W || !V || !Z) return TP_ERR_NULL;
  for (int i = 0; i < k; ++i) {
    if (!W[i] || !V[i] || (b && !b[i])) return TP_ERR_NULL;
    if (!aligned16(W[i]) || !aligned16(V[i]) || (b && !aligned16(b[i]))) return TP_ERR_ALIGN;
  }
  if (!aligned16(X) || !aligned16(Z)) return TP_ERR_ALIGN;
  return TP_OK;
}

// The forward's inputs, for the overlap check.
void forward_regions(const void* X, const void* const* W, const void* const* b, const void* const* V, int k,
                     int64_t M, int64_t H, int64_t Fk, int dtype, Regions& in) {
  const size_t e = elt_size(dtype);
  in.add(X, size_t(M) * size_t(H) * e);
  for (int i = 0; i < k; ++i) {
    in.add(W[i], size_t(H) * size_t(Fk) * e);
    in.add(V[i], size_t(Fk) * size_t(H) * e);
    if (b) in.add(b[i], size_t(Fk) * e);
  }
}

// The whole forward on a buffer `ws` that holds G shards' Y_i [M, Fk] and,
// for the literal variant, the k - 1 float32 partials after them.
int run_forward(const void* X, const void* const* W, const void* const* b, const void* const* V, int k,
                int64_t M, int64_t H, int64_t Fk, int dtype, float* Z, unsigned flags, char* ws, int G,
                hipStream_t s) {
  const bool fused = (flags & TP_FUSED_ACCUM) != 0;
  const size_t y_bytes = round_up(size_t(M) * size_t(Fk) * elt_size(dtype), kWsAlign);
  const size_t part_bytes = round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  void* Y[kMaxGroups];
  for (int j = 0; j < G; ++j) Y[j] = ws + size_t(j) * y_bytes;
  char* part_base = ws + size_t(G) * y_bytes;
  const float* parts[TP_MAX_SHARDS];
  // P_0 (or the fused sum) in Z, P_1 .. P_{k-1} after the Y_i.
  auto part = [&](int i) {
    return i == 0 ? Z : reinterpret_cast<float*>(part_base + size_t(i - 1) * part_bytes);
  };
  auto col = [&](int i0, int n) {
    return col_steps(X, W + i0, b ? b + i0 : nullptr, Y, nullptr, n, M, H, Fk, dtype, s);
  };
  int st = shard_steps(col, V, k, M, H, Fk, dtype, Y, fused, part, parts, s, G);
  if (st) return st;
  if (!fused && k > 1) return hip_status(tpmlp::launch_shard_reduce(parts, k, Z, M * H, s));
  return TP_OK;
}

// The batch of a bf16 forward step for the tile queries (shapes only).
int step_batch(int step, int n, int64_t M, int64_t H, int64_t Fk, unsigned flags, GemmBatch& g) {
  int st = check_dims(M, H, Fk);
  if (st) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  switch (step) {
    case 0: g = col_batch(nullptr, nullptr, nullptr, nullptr, nullptr, n, M, H, Fk); return TP_OK;
    case 1:
    case 2:
      if (flags & ~TP_ACCUMULATE) return TP_ERR_FLAGS;
      g = row_batch(nullptr, nullptr, nullptr, n, step == 2, M, Fk, H, (flags & TP_ACCUMULATE) != 0);
      return TP_OK;
    default: return TP_ERR_SHAPE;
  }
}

// tp_attn_core_shards with a chosen attention kernel (-1: the library's).
int attn_core_variant(int variant, const void* const* QKV, void* const* A, int n, int64_t B, int64_t S,
                      int heads, int head_dim, int dtype, unsigned flags, void* stream) {
  if (check_dtype(dtype)) return TP_ERR_DTYPE;
  if (dtype != TP_BF16) return TP_ERR_DTYPE;
  if (flags & ~TP_CAUSAL) return TP_ERR_FLAGS;
  if (n < 1 || n > TP_MAX_BATCH || heads < 1) return TP_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return TP_ERR_SHAPE;
  int st = check_attn(B, S, int64_t(heads) * head_dim, heads, 1);
  if (st) return st;
  if (B == 0 || S == 0) return TP_OK;
  if (!QKV || !A) return TP_ERR_NULL;
  const size_t M = size_t(B) * size_t(S), Hk = size_t(heads) * size_t(head_dim);
  Regions in, out;
  for (int i = 0; i < n; ++i) {
    if (!QKV[i] || !A[i]) return TP_ERR_NULL;
    if (!aligned16(QKV[i]) || !aligned16(A[i])) return TP_ERR_ALIGN;
    in.add(QKV[i], M * 3 * Hk * 2);
    out.add(A[i], M * Hk * 2);
  }
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return hip_status(tpmlp::launch_attention_bf16_variant(variant, QKV, A, n, B, S, heads, head_dim,
                                                         (flags & TP_CAUSAL) != 0, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* tp_status_string(int status) {
  switch (status) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "a required pointer is NULL";
    case TP_ERR_SHAPE:
      return "a size is out of range (H and F/k must be multiples of 8, 8 <= H, F/k <= 2^22)";
    case TP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case TP_ERR_DTYPE: return "unknown dtype (expected TP_F32 or TP_BF16)";
    case TP_ERR_WORKSPACE: return "workspace is missing or too small";
    case TP_ERR_HIP: return "a HIP launch failed";
    case TP_ERR_FLAGS: return "unknown flag bits";
    case TP_ERR_ALIAS: return "an output overlaps an input or another output";
    default: return "unknown status";
  }
}

int tp_mlp_version(void) { return 200; }

int tp_mlp_col_gelu_shards(const void* X, const void* const* W, const void* const* b, void* const* Y,
                           void* const* G, int n, int64_t M, int64_t H, int64_t Fk, int dtype,
                           void* stream) {
  return col_shards(X, W, b, Y, G, n, M, H, Fk, dtype, stream, -1);
}

int tp_mlp_col_gelu(const void* X, const void* W_i, const void* b_i, void* Y_i, int64_t M,
                    int64_t H, int64_t Fk, int dtype, void* stream) {
  return tp_mlp_col_gelu_shards(X, &W_i, b_i ? &b_i : nullptr, &Y_i, nullptr, 1, M, H, Fk, dtype,
                                stream);
}

int tp_mlp_col_gelu_save(const void* X, const void* W_i, const void* b_i, void* Y_i, void* G_i,
                         int64_t M, int64_t H, int64_t Fk, int dtype, void* stream) {
  return tp_mlp_col_gelu_shards(X, &W_i, b_i ? &b_i : nullptr, &Y_i, &G_i, 1, M, H, Fk, dtype,
                                stream);
}

int tp_mlp_row_partial_shards(const void* const* Y, const void* const* V, float* const* Z, int n,
                              int64_t M, int64_t Fk, int64_t H, int dtype, unsigned flags,
                              void* stream) {
  return row_shards(Y, V, Z, n, M, Fk, H, dtype, flags, stream, -1);
}

int tp_mlp_row_partial(const void* Y_i, const void* V_i, float* Z_i, int64_t M, int64_t Fk,
                       int64_t H, int dtype, unsigned flags, void* stream) {
  if (flags & ~TP_ACCUMULATE) return check_dtype(dtype) ? check_dtype(dtype) : TP_ERR_FLAGS;
  return tp_mlp_row_partial_shards(&Y_i, &V_i, &Z_i, 1, M, Fk, H, dtype, flags, stream);
}

int tp_shard_reduce(const float* const* Z_parts, int k, float* Z, int64_t n, void* stream) {
  if (k < 1 || k > TP_MAX_SHARDS) return TP_ERR_SHAPE;
  if (n < 0 || n > kMaxElems) return TP_ERR_SHAPE;
  if (n == 0) return TP_OK;
  if (!Z_parts || !Z) return TP_ERR_NULL;
  for (int i = 0; i < k; ++i) {
    if (!Z_parts[i]) return TP_ERR_NULL;
    if (!aligned16(Z_parts[i])) return TP_ERR_ALIGN;
  }
  if (!aligned16(Z)) return TP_ERR_ALIGN;
  const size_t nb = size_t(n) * 4;
  for (int i = 0; i < k; ++i) {
    if (Z_parts[i] == Z && i == 0) continue;
    if (overlap(Z, nb, Z_parts[i], nb)) return TP_ERR_ALIAS;
  }
  return hip_status(tpmlp::launch_shard_reduce(Z_parts, k, Z, n, static_cast<hipStream_t>(stream)));
}

size_t tp_mlp_workspace_bytes(int k, int64_t M, int64_t H, int64_t Fk, int dtype, unsigned flags) {
  if (k < 1 || k > TP_MAX_SHARDS || check_dtype(dtype) || check_dims(M, H, Fk)) return 0;
  if (flags & ~TP_FUSED_ACCUM) return 0;
  if (M == 0) return 0;
  size_t bytes = size_t(batch_size(k)) * round_up(size_t(M) * size_t(Fk) * elt_size(dtype), kWsAlign);
  if (!(flags & TP_FUSED_ACCUM)) bytes += size_t(k - 1) * round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  return bytes;
}

int tp_mlp_shard_forward(const void* X, const void* const* W, const void* const* b,
                         const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                         int dtype, void* workspace, size_t workspace_bytes, float* Z,
                         unsigned flags, void* stream) {
  int st = check_forward(X, W, b, V, k, M, H, Fk, dtype, Z, flags);
  if (st || M == 0) return st;
  const size_t need = tp_mlp_workspace_bytes(k, M, H, Fk, dtype, flags);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TP_ERR_ALIGN;
  Regions in, out;
  forward_regions(X, W, b, V, k, M, H, Fk, dtype, in);
  out.add(Z, size_t(M) * size_t(H) * 4);
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return run_forward(X, W, b, V, k, M, H, Fk, dtype, Z, flags, static_cast<char*>(workspace), batch_size(k),
                     static_cast<hipStream_t>(stream));
}

int tp_mlp_shard_forward_noalloc(const void* X, const void* const* W, const void* const* b,
                                 const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                                 int dtype, float* Z, unsigned flags, void* stream) {
  int st = check_forward(X, W, b, V, k, M, H, Fk, dtype, Z, flags);
  if (st || M == 0) return st;
  // The scratch array holds a batch of G shards' Y_i and, literal, the k - 1
  // partials: the largest G <= TP_MAX_BATCH that fits (none: TP_ERR_WORKSPACE).
  const size_t y_bytes = round_up(size_t(M) * size_t(Fk) * elt_size(dtype), kWsAlign);
  const size_t p_bytes = (flags & TP_FUSED_ACCUM) ? 0 : size_t(k - 1) * round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  const size_t cap = TP_NOALLOC_SCRATCH_BYTES;
  if (p_bytes >= cap || (cap - p_bytes) / y_bytes < 1) return TP_ERR_WORKSPACE;
  const size_t fit = (cap - p_bytes) / y_bytes;
  const int G = fit < size_t(batch_size(k)) ? int(fit) : batch_size(k);
  Regions in;
  forward_regions(X, W, b, V, k, M, H, Fk, dtype, in);
  Regions out;
  out.add(Z, size_t(M) * size_t(H) * 4);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if (tpmlp::noalloc_scratch(s, &scratch) != hipSuccess) return TP_ERR_HIP;
  // Y_i batches first, the partials after them (run_forward's layout).
  return run_forward(X, W, b, V, k, M, H, Fk, dtype, Z, flags, static_cast<char*>(scratch), G, s);
}

int tp_sp_reduce_scatter(const float* const* Z_parts, int nparts, const void* R, int r_dtype,
                         void* const* O, int out_dtype, int k, int64_t M, int64_t H, void* stream) {
  int st = check_sp(Z_parts, nparts, R, r_dtype, O, out_dtype, k, M, H);
  if (st || M == 0) return st;
  return hip_status(tpmlp::launch_sp_reduce_scatter(Z_parts, nparts, R, r_dtype == TP_BF16, O,
                                                    out_dtype == TP_BF16, k, (M / k) * H,
                                                    static_cast<hipStream_t>(stream)));
}

size_t tp_mlp_sp_workspace_bytes(int k, int64_t M, int64_t H, int64_t Fk, int dtype, unsigned flags) {
  if (k < 1 || k > TP_MAX_SHARDS || check_dtype(dtype) || check_dims(M, H, Fk)) return 0;
  if (flags & ~TP_FUSED_ACCUM) return 0;
  if (M == 0 || M % k) return 0;
  const size_t y = round_up(size_t(M) * size_t(Fk) * elt_size(dtype), kWsAlign);
  const size_t part = round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  return size_t(batch_size(k)) * y + size_t((flags & TP_FUSED_ACCUM) ? 1 : k) * part;
}

int tp_mlp_shard_forward_sp(const void* X, const void* const* W, const void* const* b,
                            const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                            int dtype, void* workspace, size_t workspace_bytes, void* const* O,
                            int out_dtype, unsigned flags, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (check_dtype(out_dtype)) return TP_ERR_DTYPE;
  if (flags & ~TP_FUSED_ACCUM) return TP_ERR_FLAGS;
  if (k < 1 || k > TP_MAX_SHARDS) return TP_ERR_SHAPE;
  if ((st = check_dims(M, H, Fk))) return st;
  if (M % k) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (!X || !W || !V || !O) return TP_ERR_NULL;
  for (int i = 0; i < k; ++i) {
    if (!W[i] || !V[i] || (b && !b[i]) || !O[i]) return TP_ERR_NULL;
    if (!aligned16(W[i]) || !aligned16(V[i]) || (b && !aligned16(b[i])) || !aligned16(O[i]))
      return TP_ERR_ALIGN;
  }
  if (!aligned16(X)) return TP_ERR_ALIGN;
  const size_t need = tp_mlp_sp_workspace_bytes(k, M, H, Fk, dtype, flags);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t nz = size_t(M) * size_t(H);
  Regions in, out;
  in.add(X, nz * e);
  for (int i = 0; i < k; ++i) {
    in.add(W[i], size_t(H) * size_t(Fk) * e);
    in.add(V[i], size_t(Fk) * size_t(H) * e);
    if (b) in.add(b[i], size_t(Fk) * e);
    out.add(O[i], nz / size_t(k) * elt_size(out_dtype));
  }
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = (flags & TP_FUSED_ACCUM) != 0;
  char* ws = static_cast<char*>(workspace);
  const int G = batch_size(k);
  const size_t y_bytes = round_up(size_t(M) * size_t(Fk) * e, kWsAlign);
  const size_t part_bytes = round_up(nz * 4, kWsAlign);
  void* Y[kMaxGroups];
  for (int j = 0; j < G; ++j) Y[j] = ws + size_t(j) * y_bytes;
  char* part_base = ws + size_t(G) * y_bytes;
  const float* parts[TP_MAX_SHARDS];
  auto part = [&](int i) { return reinterpret_cast<float*>(part_base + size_t(i) * part_bytes); };
  auto col = [&](int i0, int n) {
    return col_steps(X, W + i0, b ? b + i0 : nullptr, Y, nullptr, n, M, H, Fk, dtype, s);
  };
  if ((st = shard_steps(col, V, k, M, H, Fk, dtype, Y, fused, part, parts, s, G))) return st;
  if (fused) parts[0] = part(0);
  // The reduce-scatter over the k sequence blocks, with X as the residual.
  return hip_status(tpmlp::launch_sp_reduce_scatter(parts, fused ? 1 : k, X, dtype == TP_BF16, O,
                                                    out_dtype == TP_BF16, k, (M / k) * H, s));
}

int tp_swiglu_col_shards(const void* X, const void* const* Wg, const void* const* Wu, void* const* Y,
                         int n, int64_t M, int64_t H, int64_t Fk, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (!X || !Wg || !Wu || !Y) return TP_ERR_NULL;
  if (!aligned16(X)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * e);
  for (int i = 0; i < n; ++i) {
    if (!Wg[i] || !Wu[i] || !Y[i]) return TP_ERR_NULL;
    if (!aligned16(Wg[i]) || !aligned16(Wu[i]) || !aligned16(Y[i])) return TP_ERR_ALIGN;
    in.add(Wg[i], size_t(H) * size_t(Fk) * e);
    in.add(Wu[i], size_t(H) * size_t(Fk) * e);
    out.add(Y[i], size_t(M) * size_t(Fk) * e);
  }
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return swiglu_col_steps(X, Wg, Wu, Y, n, M, H, Fk, dtype, static_cast<hipStream_t>(stream));
}

int tp_swiglu_col(const void* X, const void* Wg_i, const void* Wu_i, void* Y_i, int64_t M, int64_t H,
                  int64_t Fk, int dtype, void* stream) {
  return tp_swiglu_col_shards(X, &Wg_i, &Wu_i, &Y_i, 1, M, H, Fk, dtype, stream);
}

int tp_swiglu_shard_forward(const void* X, const void* const* Wg, const void* const* Wu,
                            const void* const* V, int k, int64_t M, int64_t H, int64_t Fk, int dtype,
                            void* workspace, size_t workspace_bytes, float* Z, unsigned flags,
                            void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~TP_FUSED_ACCUM) return TP_ERR_FLAGS;
  if (k < 1 || k > TP_MAX_SHARDS) return TP_ERR_SHAPE;
  if ((st = check_dims(M, H, Fk))) return st;
  if (M == 0) return TP_OK;
  if (!X || !Wg || !Wu || !V || !Z) return TP_ERR_NULL;
  for (int i = 0; i < k; ++i) {
    if (!Wg[i] || !Wu[i] || !V[i]) return TP_ERR_NULL;
    if (!aligned16(Wg[i]) || !aligned16(Wu[i]) || !aligned16(V[i])) return TP_ERR_ALIGN;
  }
  if (!aligned16(X) || !aligned16(Z)) return TP_ERR_ALIGN;
  const size_t need = tp_mlp_workspace_bytes(k, M, H, Fk, dtype, flags);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t nz = size_t(M) * size_t(H) * 4;
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * e);
  for (int i = 0; i < k; ++i) {
    in.add(Wg[i], size_t(H) * size_t(Fk) * e);
    in.add(Wu[i], size_t(H) * size_t(Fk) * e);
    in.add(V[i], size_t(Fk) * size_t(H) * e);
  }
  out.add(Z, nz);
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = (flags & TP_FUSED_ACCUM) != 0;
  char* ws = static_cast<char*>(workspace);
  const int G = batch_size(k);
  const size_t y_bytes = round_up(size_t(M) * size_t(Fk) * e, kWsAlign);
  const size_t part_bytes = round_up(nz, kWsAlign);
  void* Y[kMaxGroups];
  for (int j = 0; j < G; ++j) Y[j] = ws + size_t(j) * y_bytes;
  char* part_base = ws + size_t(G) * y_bytes;
  const float* parts[TP_MAX_SHARDS];
  auto part = [&](int i) {
    return i == 0 ? Z : reinterpret_cast<float*>(part_base + size_t(i - 1) * part_bytes);
  };
  auto col = [&](int i0, int n) { return swiglu_col_steps(X, Wg + i0, Wu + i0, Y, n, M, H, Fk, dtype, s); };
  if ((st = shard_steps(col, V, k, M, H, Fk, dtype, Y, fused, part, parts, s, G))) return st;
  if (!fused && k > 1) return hip_status(tpmlp::launch_shard_reduce(parts, k, Z, M * H, s));
  return TP_OK;
}

int tp_attn_qkv_shards(const void* X, const void* const* Wqkv, const void* const* bqkv, void* const* QKV,
                       int n, int64_t M, int64_t H, int64_t Hk, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, H, Hk))) return st;
  if (3 * Hk > kMaxLd) return TP_ERR_SHAPE;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (!X || !Wqkv || !QKV) return TP_ERR_NULL;
  if (!aligned16(X)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * e);
  for (int i = 0; i < n; ++i) {
    if (!Wqkv[i] || !QKV[i] || (bqkv && !bqkv[i])) return TP_ERR_NULL;
    if (!aligned16(Wqkv[i]) || !aligned16(QKV[i]) || (bqkv && !aligned16(bqkv[i]))) return TP_ERR_ALIGN;
    in.add(Wqkv[i], size_t(H) * size_t(3 * Hk) * e);
    if (bqkv) in.add(bqkv[i], size_t(3 * Hk) * e);
    out.add(QKV[i], size_t(M) * size_t(3 * Hk) * e);
  }
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return qkv_steps(X, Wqkv, bqkv, QKV, n, M, H, Hk, dtype, static_cast<hipStream_t>(stream));
}

int tp_attn_core_shards(const void* const* QKV, void* const* A, int n, int64_t B, int64_t S, int heads,
                        int head_dim, int dtype, unsigned flags, void* stream) {
  return attn_core_variant(-1, QKV, A, n, B, S, heads, head_dim, dtype, flags, stream);
}

size_t tp_attn_workspace_bytes(int k, int64_t B, int64_t S, int64_t H, int n_heads, int dtype, unsigned flags) {
  if (check_dtype(dtype) || dtype != TP_BF16 || check_attn(B, S, H, n_heads, k)) return 0;
  if (flags & ~(TP_FUSED_ACCUM | TP_CAUSAL)) return 0;
  const int64_t M = B * S;
  if (M == 0) return 0;
  const int64_t Hk = H / n_heads * (n_heads / k);
  const size_t qkv = round_up(size_t(M) * size_t(3 * Hk) * 2, kWsAlign);
  const size_t a = round_up(size_t(M) * size_t(Hk) * 2, kWsAlign);
  size_t bytes = size_t(batch_size(k)) * (qkv + a);
  if (!(flags & TP_FUSED_ACCUM)) bytes += size_t(k - 1) * round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  return bytes;
}

int tp_attn_shard_forward(const void* X, const void* const* Wqkv, const void* const* bqkv,
                          const void* const* Wo, int k, int64_t B, int64_t S, int64_t H, int n_heads,
                          int dtype, void* workspace, size_t workspace_bytes, float* Z, unsigned flags,
                          void* stream) {
  if (check_dtype(dtype) || dtype != TP_BF16) return TP_ERR_DTYPE;
  if (flags & ~(TP_FUSED_ACCUM | TP_CAUSAL)) return TP_ERR_FLAGS;
  int st = check_attn(B, S, H, n_heads, k);
  if (st) return st;
  const int64_t M = B * S;
  if (M == 0) return TP_OK;
  const int64_t d = H / n_heads, hk = n_heads / k, Hk = d * hk;
  if (!X || !Wqkv || !Wo || !Z) return TP_ERR_NULL;
  for (int i = 0; i < k; ++i) {
    if (!Wqkv[i] || !Wo[i] || (bqkv && !bqkv[i])) return TP_ERR_NULL;
    if (!aligned16(Wqkv[i]) || !aligned16(Wo[i]) || (bqkv && !aligned16(bqkv[i]))) return TP_ERR_ALIGN;
  }
  if (!aligned16(X) || !aligned16(Z)) return TP_ERR_ALIGN;
  const size_t need = tp_attn_workspace_bytes(k, B, S, H, n_heads, dtype, flags);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t nz = size_t(M) * size_t(H) * 4;
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * 2);
  for (int i = 0; i < k; ++i) {
    in.add(Wqkv[i], size_t(H) * size_t(3 * Hk) * 2);
    in.add(Wo[i], size_t(Hk) * size_t(H) * 2);
    if (bqkv) in.add(bqkv[i], size_t(3 * Hk) * 2);
  }
  out.add(Z, nz);
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = (flags & TP_FUSED_ACCUM) != 0;
  const bool causal = (flags & TP_CAUSAL) != 0;
  char* ws = static_cast<char*>(workspace);
  const int G = batch_size(k);
  const size_t qkv_bytes = round_up(size_t(M) * size_t(3 * Hk) * 2, kWsAlign);
  const size_t a_bytes = round_up(size_t(M) * size_t(Hk) * 2, kWsAlign);
  const size_t part_bytes = round_up(nz, kWsAlign);
  void* QKV[kMaxGroups];
  void* A[kMaxGroups];
  for (int j = 0; j < G; ++j) {
    QKV[j] = ws + size_t(j) * qkv_bytes;
    A[j] = ws + size_t(G) * qkv_bytes + size_t(j) * a_bytes;
  }
  char* part_base = ws + size_t(G) * (qkv_bytes + a_bytes);
  const float* parts[TP_MAX_SHARDS];
  auto part = [&](int i) {
    return i == 0 ? Z : reinterpret_cast<float*>(part_base + size_t(i - 1) * part_bytes);
  };
  // The "column step" of a batch: the head-split projection, then each
  // shard's heads' attention into A (the row step's input).
  auto col = [&](int i0, int n) {
    int r = qkv_steps(X, Wqkv + i0, bqkv ? bqkv + i0 : nullptr, QKV, n, M, H, Hk, dtype, s);
    if (r) return r;
    return hip_status(tpmlp::launch_attention_bf16(QKV, A, n, B, S, (int)hk, (int)d, causal, s));
  };
  if ((st = shard_steps(col, Wo, k, M, H, Hk, dtype, A, fused, part, parts, s, G))) return st;
  if (!fused && k > 1) return hip_status(tpmlp::launch_shard_reduce(parts, k, Z, M * H, s));
  return TP_OK;
}

int tp_mlp_grad_act_shards(const void* dZ, const void* const* V, const void* const* G,
                           void* const* dA, int n, int64_t M, int64_t H, int64_t Fk, int dtype,
                           void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  if (!dZ || !V || !G || !dA) return TP_ERR_NULL;
  if (!aligned16(dZ)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t na = size_t(M) * size_t(Fk) * e;
  Regions in, out;
  in.add(dZ, size_t(M) * size_t(H) * e);
  for (int i = 0; i < n; ++i) {
    if (!V[i] || !G[i] || !dA[i]) return TP_ERR_NULL;
    if (!aligned16(V[i]) || !aligned16(G[i]) || !aligned16(dA[i])) return TP_ERR_ALIGN;
    in.add(V[i], size_t(Fk) * size_t(H) * e);
    out.add(dA[i], na);
  }
  // G[i] may be dA[i] itself, but no other output
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < out.n; ++j)
      if (!(j == i && G[i] == dA[i]) && overlap(G[i], na, out.r[j].p, out.r[j].n)) return TP_ERR_ALIAS;
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return act_grad_steps(dZ, V, G, dA, n, M, H, Fk, dtype, static_cast<hipStream_t>(stream));
}

int tp_mlp_grad_act(const void* dZ, const void* V_i, const void* G_i, void* dA_i, int64_t M,
                    int64_t H, int64_t Fk, int dtype, void* stream) {
  return tp_mlp_grad_act_shards(dZ, &V_i, &G_i, &dA_i, 1, M, H, Fk, dtype, stream);
}

size_t tp_mlp_grad_weight_workspace_bytes_shards(int n, int64_t M, int64_t H, int64_t Fk,
                                                 int dtype) {
  if (n < 1 || n > TP_MAX_BATCH || check_dtype(dtype) || check_dims(M, H, Fk)) return 0;
  return grad_weight_ws(n, M, H, Fk, dtype);
}

size_t tp_mlp_grad_weight_workspace_bytes(int64_t M, int64_t H, int64_t Fk, int dtype) {
  return tp_mlp_grad_weight_workspace_bytes_shards(1, M, H, Fk, dtype);
}

int tp_mlp_grad_row_weight_shards(const void* const* Y, const void* dZ, float* const* dV, int n,
                                  int64_t M, int64_t Fk, int64_t H, int dtype, void* workspace,
                                  size_t workspace_bytes, unsigned flags, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~TP_GRAD_ACCUMULATE) return TP_ERR_FLAGS;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (!Y || !dV || (M > 0 && !dZ)) return TP_ERR_NULL;
  if (!aligned16(dZ)) return TP_ERR_ALIGN;
  const size_t need = grad_weight_ws(n, M, H, Fk, dtype);
  if (need && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  Regions in, out;
  in.add(dZ, size_t(M) * size_t(H) * e);
  for (int i = 0; i < n; ++i) {
    if (!dV[i] || (M > 0 && !Y[i])) return TP_ERR_NULL;
    if (!aligned16(Y[i]) || !aligned16(dV[i])) return TP_ERR_ALIGN;
    in.add(Y[i], size_t(M) * size_t(Fk) * e);
    out.add(dV[i], size_t(Fk) * size_t(H) * 4);
  }
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return row_weight_steps(Y, dZ, dV, n, M, Fk, H, dtype, workspace,
                          (flags & TP_GRAD_ACCUMULATE) != 0, static_cast<hipStream_t>(stream));
}

int tp_mlp_grad_row_weight(const void* Y_i, const void* dZ, float* dV_i, int64_t M, int64_t Fk,
                           int64_t H, int dtype, void* workspace, size_t workspace_bytes,
                           unsigned flags, void* stream) {
  return tp_mlp_grad_row_weight_shards(&Y_i, dZ, &dV_i, 1, M, Fk, H, dtype, workspace,
                                       workspace_bytes, flags, stream);
}

int tp_mlp_grad_col_weight_shards(const void* X, const void* const* dA, float* const* dW,
                                  float* const* db, int n, int64_t M, int64_t H, int64_t Fk,
                                  int dtype, void* workspace, size_t workspace_bytes,
                                  unsigned flags, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~TP_GRAD_ACCUMULATE) return TP_ERR_FLAGS;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (!dA || !dW || (M > 0 && !X)) return TP_ERR_NULL;
  if (!aligned16(X)) return TP_ERR_ALIGN;
  const size_t need = grad_weight_ws(n, M, H, Fk, dtype);
  if (need && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * e);
  for (int i = 0; i < n; ++i) {
    if (!dW[i] || (M > 0 && !dA[i]) || (db && !db[i])) return TP_ERR_NULL;
    if (!aligned16(dA[i]) || !aligned16(dW[i]) || (db && !aligned16(db[i]))) return TP_ERR_ALIGN;
    in.add(dA[i], size_t(M) * size_t(Fk) * e);
    out.add(dW[i], size_t(H) * size_t(Fk) * 4);
    if (db) out.add(db[i], size_t(Fk) * 4);
  }
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return col_weight_steps(X, dA, dW, db, n, M, H, Fk, dtype, workspace,
                          (flags & TP_GRAD_ACCUMULATE) != 0, static_cast<hipStream_t>(stream));
}

int tp_mlp_grad_col_weight(const void* X, const void* dA_i, float* dW_i, float* db_i, int64_t M,
                           int64_t H, int64_t Fk, int dtype, void* workspace,
                           size_t workspace_bytes, unsigned flags, void* stream) {
  return tp_mlp_grad_col_weight_shards(X, &dA_i, &dW_i, db_i ? &db_i : nullptr, 1, M, H, Fk, dtype,
                                       workspace, workspace_bytes, flags, stream);
}

int tp_mlp_grad_input_shards(const void* const* dA, const void* const* W, float* const* dX, int n,
                             int64_t M, int64_t Fk, int64_t H, int dtype, unsigned flags,
                             void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~(TP_ACCUMULATE | TP_SUM_SHARDS)) return TP_ERR_FLAGS;
  if ((st = check_dims(M, H, Fk))) return st;
  if (n < 1 || n > TP_MAX_BATCH) return TP_ERR_SHAPE;
  if (M == 0) return TP_OK;
  const bool sum = (flags & TP_SUM_SHARDS) != 0;
  if (!dA || !W || !dX) return TP_ERR_NULL;
  const size_t e = elt_size(dtype);
  Regions in, out;
  for (int i = 0; i < n; ++i) {
    if (!dA[i] || !W[i] || ((!sum || i == 0) && !dX[i])) return TP_ERR_NULL;
    if (!aligned16(dA[i]) || !aligned16(W[i]) || ((!sum || i == 0) && !aligned16(dX[i])))
      return TP_ERR_ALIGN;
    in.add(dA[i], size_t(M) * size_t(Fk) * e);
    in.add(W[i], size_t(H) * size_t(Fk) * e);
    if (!sum || i == 0) out.add(dX[i], size_t(M) * size_t(H) * 4);
  }
  if (any_overlap(out, in)) return TP_ERR_ALIAS;
  return input_grad_steps(dA, W, dX, n, sum, M, Fk, H, dtype, (flags & TP_ACCUMULATE) != 0,
                          static_cast<hipStream_t>(stream));
}

int tp_mlp_grad_input_partial(const void* dA_i, const void* W_i, float* dX_i, int64_t M,
                              int64_t Fk, int64_t H, int dtype, unsigned flags, void* stream) {
  if (flags & ~TP_ACCUMULATE) return check_dtype(dtype) ? check_dtype(dtype) : TP_ERR_FLAGS;
  return tp_mlp_grad_input_shards(&dA_i, &W_i, &dX_i, 1, M, Fk, H, dtype, flags, stream);
}

size_t tp_mlp_backward_workspace_bytes(int k, int64_t M, int64_t H, int64_t Fk, int dtype,
                                       unsigned flags) {
  if (k < 1 || k > TP_MAX_SHARDS || check_dtype(dtype) || check_dims(M, H, Fk)) return 0;
  if (flags & ~(TP_FUSED_ACCUM | TP_GRAD_ACCUMULATE)) return 0;
  const size_t act = round_up(size_t(M) * size_t(Fk) * elt_size(dtype), kWsAlign);
  const int G = batch_size(k);
  size_t bytes = 2 * size_t(G) * act + grad_weight_ws(G, M, H, Fk, dtype);
  if (!(flags & TP_FUSED_ACCUM)) bytes += size_t(k - 1) * round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  if (backward_transposes(M, dtype)) bytes += 2 * size_t(G) * round_up(size_t(H) * size_t(Fk) * 2, kWsAlign);
  return bytes;
}

int tp_mlp_shard_backward(const void* X, const void* const* W, const void* const* b,
                          const void* const* V, const void* dZ, int k, int64_t M, int64_t H,
                          int64_t Fk, int dtype, void* workspace, size_t workspace_bytes,
                          float* dX, float* const* dW, float* const* db, float* const* dV,
                          unsigned flags, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~(TP_FUSED_ACCUM | TP_GRAD_ACCUMULATE)) return TP_ERR_FLAGS;
  if (k < 1 || k > TP_MAX_SHARDS) return TP_ERR_SHAPE;
  if ((st = check_dims(M, H, Fk))) return st;
  if (!W || !V || !dW || !dV || (M > 0 && (!X || !dZ || !dX))) return TP_ERR_NULL;
  for (int i = 0; i < k; ++i) {
    if (!W[i] || !V[i] || !dW[i] || !dV[i] || (b && !b[i]) || (db && !db[i])) return TP_ERR_NULL;
    if (!aligned16(W[i]) || !aligned16(V[i]) || !aligned16(dW[i]) || !aligned16(dV[i]) ||
        (b && !aligned16(b[i])) || (db && !aligned16(db[i])))
      return TP_ERR_ALIGN;
  }
  if (!aligned16(X) || !aligned16(dZ) || (dX && !aligned16(dX))) return TP_ERR_ALIGN;
  const size_t need = tp_mlp_backward_workspace_bytes(k, M, H, Fk, dtype, flags);
  if (need && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t nx = size_t(M) * size_t(H) * 4;
  Regions in, out;
  in.add(X, size_t(M) * size_t(H) * e);
  in.add(dZ, size_t(M) * size_t(H) * e);
  for (int i = 0; i < k; ++i) {
    in.add(W[i], size_t(H) * size_t(Fk) * e);
    in.add(V[i], size_t(Fk) * size_t(H) * e);
    if (b) in.add(b[i], size_t(Fk) * e);
    out.add(dW[i], size_t(H) * size_t(Fk) * 4);
    out.add(dV[i], size_t(Fk) * size_t(H) * 4);
    if (db) out.add(db[i], size_t(Fk) * 4);
  }
  out.add(dX, nx);
  out.add(workspace, need);
  if (any_overlap(out, in)) return TP_ERR_ALIAS;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = (flags & TP_FUSED_ACCUM) != 0;
  const bool acc_grads = (flags & TP_GRAD_ACCUMULATE) != 0;
  char* ws = static_cast<char*>(workspace);
  const int G = batch_size(k);
  const size_t act = round_up(size_t(M) * size_t(Fk) * e, kWsAlign);
  void* Y[kMaxGroups];
  void* Gb[kMaxGroups];  // G_i, then dA_i in place
  for (int j = 0; j < G; ++j) {
    Y[j] = ws + size_t(j) * act;
    Gb[j] = ws + size_t(G + j) * act;
  }
  void* wws = ws + 2 * size_t(G) * act;
  const size_t part_bytes = round_up(nx, kWsAlign);
  char* part_base = ws + 2 * size_t(G) * act + grad_weight_ws(G, M, H, Fk, dtype);
  const float* parts[TP_MAX_SHARDS];
  float* P[kMaxGroups];
  // Transposed weights (bf16, M large enough): Vt_i [H, Fk] and Wt_i [Fk, H]
  // after the partials, so that dZ V_i^T and dA_i W_i^T run on the NN path.
  const bool tr = backward_transposes(M, dtype);
  void* Vt[kMaxGroups];
  void* Wt[kMaxGroups];
  if (tr) {
    const size_t wbytes = round_up(size_t(H) * size_t(Fk) * 2, kWsAlign);
    char* tw = part_base + (fused ? 0 : size_t(k - 1) * part_bytes);
    for (int j = 0; j < G; ++j) {
      Vt[j] = tw + size_t(j) * wbytes;
      Wt[j] = tw + size_t(G + j) * wbytes;
    }
  }

  for (int i0 = 0; i0 < k; i0 += G) {
    const int n = k - i0 < G ? k - i0 : G;
    if (M > 0) {
      // Recompute Y_i and G_i, then dA_i = (dZ V_i^T) * G_i in place.
      if ((st = col_steps(X, W + i0, b ? b + i0 : nullptr, Y, Gb, n, M, H, Fk, dtype, s))) return st;
      if (tr) {
        if ((st = hip_status(tpmlp::launch_transpose_bf16(V + i0, Vt, n, Fk, H, s)))) return st;
        if ((st = act_grad_nn_steps(dZ, Vt, Gb, Gb, n, M, H, Fk, dtype, s))) return st;
      } else if ((st = act_grad_steps(dZ, V + i0, Gb, Gb, n, M, H, Fk, dtype, s))) {
        return st;
      }
    }
    if ((st = row_weight_steps(Y, dZ, dV + i0, n, M, Fk, H, dtype, wws, acc_grads, s))) return st;
    if ((st = col_weight_steps(X, Gb, dW + i0, db ? db + i0 : nullptr, n, M, H, Fk, dtype, wws,
                               acc_grads, s)))
      return st;
    if (M == 0) continue;
    // dX_i = dA_i W_i^T: on the NN path through Wt_i (the row step's GEMM), or
    // with W_i read as its transpose.
    if (tr && (st = hip_status(tpmlp::launch_transpose_bf16(W + i0, Wt, n, H, Fk, s)))) return st;
    auto input_grads = [&](float* const* out, bool sum, bool accumulate) {
      return tr ? row_steps(Gb, Wt, out, n, sum, M, Fk, H, dtype, accumulate, s)
                : input_grad_steps(Gb, W + i0, out, n, sum, M, Fk, H, dtype, accumulate, s);
    };
    if (fused) {
      P[0] = dX;
      if ((st = input_grads(P, true, i0 > 0))) return st;
    } else {
      for (int j = 0; j < n; ++j) {
        const int i = i0 + j;
        P[j] = i == 0 ? dX : reinterpret_cast<float*>(part_base + size_t(i - 1) * part_bytes);
        parts[i] = P[j];
      }
      if ((st = input_grads(P, false, false))) return st;
    }
  }
  if (M > 0 && !fused && k > 1) return hip_status(tpmlp::launch_shard_reduce(parts, k, dX, M * H, s));
  return TP_OK;
}

int tp_gemm_tiles(int tile, int* info) {
  const int count = tpmlp::gemm_bf16_tile_count();
  if (tile >= 0 && tile < count && info) tpmlp::gemm_bf16_tile_shape(tile, info);
  return count;
}

int tp_mlp_step_tile(int step, int n, int64_t M, int64_t H, int64_t Fk) {
  GemmBatch g;
  const int st = step_batch(step, n, M, H, Fk, 0, g);
  return st ? st : tpmlp::gemm_bf16_batch_tile(g);
}

int tp_mlp_col_gelu_shards_tile(int tile, const void* X, const void* const* W, const void* const* b,
                                void* const* Y, int n, int64_t M, int64_t H, int64_t Fk, void* stream) {
  GemmBatch g;
  const int st = step_batch(0, n, M, H, Fk, 0, g);
  if (st) return st;
  if (!tpmlp::gemm_bf16_tile_can_run(tile, g)) return TP_ERR_SHAPE;
  return col_shards(X, W, b, Y, nullptr, n, M, H, Fk, TP_BF16, stream, tile);
}

int tp_mlp_row_partial_shards_tile(int tile, const void* const* Y, const void* const* V, float* const* Z,
                                   int n, int64_t M, int64_t Fk, int64_t H, unsigned flags, void* stream) {
  if (flags & ~(TP_ACCUMULATE | TP_SUM_SHARDS)) return TP_ERR_FLAGS;
  GemmBatch g;
  const int st = step_batch((flags & TP_SUM_SHARDS) ? 2 : 1, n, M, H, Fk, flags & TP_ACCUMULATE, g);
  if (st) return st;
  if (!tpmlp::gemm_bf16_tile_can_run(tile, g)) return TP_ERR_SHAPE;
  return row_shards(Y, V, Z, n, M, Fk, H, TP_BF16, flags, stream, tile);
}

int tp_attn_core_shards_variant(int variant, const void* const* QKV, void* const* A, int n, int64_t B, int64_t S,
                                int heads, int head_dim, int dtype, unsigned flags, void* stream) {
  if (variant < 0 || variant > 1) return TP_ERR_SHAPE;
  return attn_core_variant(variant, QKV, A, n, B, S, heads, head_dim, dtype, flags, stream);
}

}  // extern "C"
