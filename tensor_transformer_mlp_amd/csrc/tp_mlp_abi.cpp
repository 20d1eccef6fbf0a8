// C ABI of libtpmlp.so (declared in include/tp_mlp.h): argument checks, the
// shard loop and the workspace layout.  Every check runs on the host before
// the first HIP call, so a rejected call launches nothing.
#include "tp_mlp.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_mlp_kernels.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elt_size(int dtype) { return dtype == TP_BF16 ? 2 : 4; }

// Shape rules shared by every entry point.  M may be 0.
int check_dims(int64_t M, int64_t H, int64_t Fk) {
  if (M < 0 || M > kMaxDim) return TP_ERR_SHAPE;
  if (H < 8 || H > kMaxDim || H % 8) return TP_ERR_SHAPE;
  if (Fk < 8 || Fk > kMaxDim || Fk % 8) return TP_ERR_SHAPE;
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

int hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

int col_gelu_checked(const void* X, const void* W_i, const void* b_i, void* Y_i, int64_t M,
                     int64_t H, int64_t Fk, int dtype, hipStream_t s) {
  if (dtype == TP_BF16)
    return hip_status(tpmlp::launch_gemm_bf16(static_cast<const uint16_t*>(X),
                                              static_cast<const uint16_t*>(W_i),
                                              static_cast<const uint16_t*>(b_i), Y_i, M, Fk, H,
                                              tpmlp::kEpiBiasGelu, s));
  return hip_status(tpmlp::launch_gemm_f32(static_cast<const float*>(X),
                                           static_cast<const float*>(W_i),
                                           static_cast<const float*>(b_i), Y_i, M, Fk, H,
                                           tpmlp::kEpiBiasGelu, s));
}

int row_partial_checked(const void* Y_i, const void* V_i, float* Z_i, int64_t M, int64_t Fk,
                        int64_t H, int dtype, bool accumulate, hipStream_t s) {
  const tpmlp::Epilogue epi = accumulate ? tpmlp::kEpiAccumF32 : tpmlp::kEpiStoreF32;
  if (dtype == TP_BF16)
    return hip_status(tpmlp::launch_gemm_bf16(static_cast<const uint16_t*>(Y_i),
                                              static_cast<const uint16_t*>(V_i), nullptr, Z_i, M,
                                              H, Fk, epi, s));
  return hip_status(tpmlp::launch_gemm_f32(static_cast<const float*>(Y_i),
                                           static_cast<const float*>(V_i), nullptr, Z_i, M, H, Fk,
                                           epi, s));
}

}  // namespace

extern "C" {

const char* tp_status_string(int status) {
  switch (status) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "a required pointer is NULL";
    case TP_ERR_SHAPE: return "a size is out of range (H and F/k must be multiples of 8, >= 8)";
    case TP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case TP_ERR_DTYPE: return "unknown dtype (expected TP_F32 or TP_BF16)";
    case TP_ERR_WORKSPACE: return "workspace is missing or too small";
    case TP_ERR_HIP: return "a HIP launch failed";
    case TP_ERR_FLAGS: return "unknown flag bits";
    case TP_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
  }
}

int tp_mlp_version(void) { return 100; }

int tp_mlp_col_gelu(const void* X, const void* W_i, const void* b_i, void* Y_i, int64_t M,
                    int64_t H, int64_t Fk, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if ((st = check_dims(M, H, Fk))) return st;
  if (M == 0) return TP_OK;
  if (!X || !W_i || !Y_i) return TP_ERR_NULL;
  if (!aligned16(X) || !aligned16(W_i) || !aligned16(Y_i) || (b_i && !aligned16(b_i)))
    return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t ny = size_t(M) * size_t(Fk) * e;
  if (overlap(Y_i, ny, X, size_t(M) * size_t(H) * e) ||
      overlap(Y_i, ny, W_i, size_t(H) * size_t(Fk) * e) ||
      (b_i && overlap(Y_i, ny, b_i, size_t(Fk) * e)))
    return TP_ERR_ALIAS;
  return col_gelu_checked(X, W_i, b_i, Y_i, M, H, Fk, dtype, static_cast<hipStream_t>(stream));
}

int tp_mlp_row_partial(const void* Y_i, const void* V_i, float* Z_i, int64_t M, int64_t Fk,
                       int64_t H, int dtype, unsigned flags, void* stream) {
  int st = check_dtype(dtype);
  if (st) return st;
  if (flags & ~TP_ACCUMULATE) return TP_ERR_FLAGS;
  if ((st = check_dims(M, H, Fk))) return st;
  if (M == 0) return TP_OK;
  if (!Y_i || !V_i || !Z_i) return TP_ERR_NULL;
  if (!aligned16(Y_i) || !aligned16(V_i) || !aligned16(Z_i)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t nz = size_t(M) * size_t(H) * 4;
  if (overlap(Z_i, nz, Y_i, size_t(M) * size_t(Fk) * e) ||
      overlap(Z_i, nz, V_i, size_t(Fk) * size_t(H) * e))
    return TP_ERR_ALIAS;
  return row_partial_checked(Y_i, V_i, Z_i, M, Fk, H, dtype, (flags & TP_ACCUMULATE) != 0,
                             static_cast<hipStream_t>(stream));
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
  size_t bytes = round_up(size_t(M) * size_t(Fk) * elt_size(dtype), kWsAlign);
  if (!(flags & TP_FUSED_ACCUM)) bytes += size_t(k - 1) * round_up(size_t(M) * size_t(H) * 4, kWsAlign);
  return bytes;
}

int tp_mlp_shard_forward(const void* X, const void* const* W, const void* const* b,
                         const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                         int dtype, void* workspace, size_t workspace_bytes, float* Z,
                         unsigned flags, void* stream) {
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
  const size_t need = tp_mlp_workspace_bytes(k, M, H, Fk, dtype, flags);
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  if (!aligned16(workspace)) return TP_ERR_ALIGN;
  const size_t e = elt_size(dtype);
  const size_t nz = size_t(M) * size_t(H) * 4;
  if (overlap(Z, nz, X, size_t(M) * size_t(H) * e) || overlap(Z, nz, workspace, need))
    return TP_ERR_ALIAS;
  if (overlap(workspace, need, X, size_t(M) * size_t(H) * e)) return TP_ERR_ALIAS;
  for (int i = 0; i < k; ++i) {
    const size_t nw = size_t(H) * size_t(Fk) * e;
    if (overlap(Z, nz, W[i], nw) || overlap(Z, nz, V[i], nw) ||
        overlap(workspace, need, W[i], nw) || overlap(workspace, need, V[i], nw) ||
        (b && (overlap(Z, nz, b[i], size_t(Fk) * e) || overlap(workspace, need, b[i], size_t(Fk) * e))))
      return TP_ERR_ALIAS;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fused = (flags & TP_FUSED_ACCUM) != 0;
  char* ws = static_cast<char*>(workspace);
  void* Y = ws;
  const size_t y_bytes = round_up(size_t(M) * size_t(Fk) * e, kWsAlign);
  const size_t part_bytes = round_up(nz, kWsAlign);
  const float* parts[TP_MAX_SHARDS];

  for (int i = 0; i < k; ++i) {
    // Column-parallel linear + bias + GeLU of shard i into the shared Y buffer.
    if ((st = col_gelu_checked(X, W[i], b ? b[i] : nullptr, Y, M, H, Fk, dtype, s))) return st;
    // Row-parallel partial of shard i.
    float* P;
    bool accumulate = false;
    if (i == 0) {
      P = Z;
    } else if (fused) {
      P = Z;
      accumulate = true;
    } else {
      P = reinterpret_cast<float*>(ws + y_bytes + size_t(i - 1) * part_bytes);
    }
    parts[i] = P;
    if ((st = row_partial_checked(Y, V[i], P, M, Fk, H, dtype, accumulate, s))) return st;
  }
  if (!fused && k > 1)
    return hip_status(tpmlp::launch_shard_reduce(parts, k, Z, M * H, s));
  return TP_OK;
}

}  // extern "C"
