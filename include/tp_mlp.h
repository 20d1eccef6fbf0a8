/*
 * tp_mlp.h — C ABI of libtpmlp.so: the forward pass of one Megatron-style
 * tensor-parallel MLP block, every shard of it on one AMD Instinct MI355X
 * (gfx950).
 *
 * The block (the first linear layer split by columns, the second by rows, one
 * all-reduce per MLP; "千亿参数模型如何拆分到多张GPU上训练", 张量并行 section,
 * 方案一 and 方案二; "大模型分布式并行策略详解：TP、DP、PP、CP、EP核心原理与实战"
 * §4.1; the ColumnParallelLinear and RowParallelLinear classes of
 * "AI大模型分布式训练：张量并行与流水线并行深度实践" §2.1-2.2):
 *
 *     Y_i = GeLU(X W_i + b_i)        column-parallel linear + activation
 *     Z_i = Y_i V_i                  row-parallel linear (a partial sum)
 *     Z   = Z_0 + ... + Z_{k-1}      the all-reduce SUM
 *
 * with GeLU(x) = x * Phi(x) (the erf form, not the tanh approximation).
 * Here the k shards run one after another on one GPU and the all-reduce is an
 * on-device sum of the k fp32 partials.
 *
 * Layout.  Every matrix is dense, row-major, [rows, cols], contiguous:
 *   X   [M, H]     activations, M = batch * sequence
 *   W_i [H, Fk]    columns [i*Fk, (i+1)*Fk) of the full W [H, F], Fk = F / k
 *   b_i [Fk]       entries [i*Fk, (i+1)*Fk) of the full bias b [F]
 *   Y_i [M, Fk]    in the input dtype
 *   V_i [Fk, H]    rows [i*Fk, (i+1)*Fk) of the full V [F, H]
 *   Z_i, Z [M, H]  always float32
 * Weights are stored [in, out] (X W, not X W^T).
 *
 * Types.  TP_BF16: X, W_i, b_i, V_i and Y_i are bfloat16; products accumulate
 * in float32; bias and GeLU are applied in float32 to the accumulator and the
 * result is rounded to nearest-even bfloat16.  TP_F32: everything float32.
 * Z_i and Z are float32 in both cases.
 *
 * Constraints.  H and Fk are multiples of 8 and at least 8; M >= 0 (M == 0 is
 * a no-op that returns TP_OK); 1 <= k <= TP_MAX_SHARDS; M, H, Fk < 2^31 and
 * each matrix holds fewer than 2^40 elements; every pointer is 16-byte
 * aligned.  Outputs must not overlap inputs unless stated.
 *
 * Ownership.  The caller owns every buffer (device memory unless stated).  The
 * library never allocates, frees or synchronises; it keeps no state between
 * calls and is safe to call from several threads on different streams.
 *
 * Errors.  Every argument is checked on the host before any HIP call; a bad
 * argument returns a negative TP_ERR_* code and launches nothing.  A failed
 * launch returns TP_ERR_HIP.  Work is asynchronous on `stream` (a hipStream_t;
 * NULL is the default stream), so a fault inside a kernel surfaces at the
 * caller's next synchronisation.
 */
#ifndef TP_MLP_H_
#define TP_MLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
#define TP_F32 0
#define TP_BF16 1

/* Status codes. */
#define TP_OK 0
#define TP_ERR_NULL (-1)      /* a required pointer is NULL */
#define TP_ERR_SHAPE (-2)     /* a size is out of range or not a multiple of 8 */
#define TP_ERR_ALIGN (-3)     /* a pointer is not 16-byte aligned */
#define TP_ERR_DTYPE (-4)     /* unknown element type */
#define TP_ERR_WORKSPACE (-5) /* workspace missing or too small */
#define TP_ERR_HIP (-6)       /* a HIP launch failed */
#define TP_ERR_FLAGS (-7)     /* unknown flag bits */
#define TP_ERR_ALIAS (-8)     /* an output overlaps an input it may not overlap */

#define TP_MAX_SHARDS 64

/* Flags. */
#define TP_ACCUMULATE 1u  /* tp_mlp_row_partial: Z_i += Y_i V_i instead of Z_i = Y_i V_i */
#define TP_FUSED_ACCUM 1u /* tp_mlp_shard_forward: fold the shard sum into the row GEMMs */

/*
 * Column-parallel linear + bias + GeLU of one shard (ColumnParallelLinear
 * forward, "AI大模型分布式训练：张量并行与流水线并行深度实践" §2.1, followed by the
 * per-shard activation of "千亿参数模型如何拆分到多张GPU上训练" 方案一):
 *
 *   Y_i[m, j] = GeLU( sum_h X[m, h] * W_i[h, j] + b_i[j] )
 *
 * X [M, H], W_i [H, Fk], b_i [Fk] (NULL means no bias), Y_i [M, Fk], all of
 * type `dtype`.  Y_i must not overlap X, W_i or b_i.
 */
int tp_mlp_col_gelu(const void* X, const void* W_i, const void* b_i, void* Y_i, int64_t M,
                    int64_t H, int64_t Fk, int dtype, void* stream);

/*
 * Row-parallel linear of one shard, the partial product that the all-reduce
 * sums (RowParallelLinear, §2.2 of the page above):
 *
 *   Z_i[m, n] = sum_j Y_i[m, j] * V_i[j, n]            (flags = 0)
 *   Z_i[m, n] = Z_i[m, n] + sum_j Y_i[m, j] * V_i[j, n] (flags = TP_ACCUMULATE)
 *
 * Y_i [M, Fk] and V_i [Fk, H] of type `dtype`; Z_i [M, H] float32, which must
 * not overlap Y_i or V_i.  With TP_ACCUMULATE the product is formed in
 * float32 and then added to the value already in Z_i (one rounding per add).
 */
int tp_mlp_row_partial(const void* Y_i, const void* V_i, float* Z_i, int64_t M, int64_t Fk,
                       int64_t H, int dtype, unsigned flags, void* stream);

/*
 * The all-reduce SUM of the k partials, on one device
 * ("dist.all_reduce(partial, op=SUM)", §2.2 of the page above):
 *
 *   Z[e] = ((Z_parts[0][e] + Z_parts[1][e]) + Z_parts[2][e]) + ...   0 <= e < n
 *
 * float32, summed left to right so that the result is deterministic.
 * `Z_parts` is a HOST array of k device pointers.  Z may be Z_parts[0] itself
 * (in place) but must not overlap any other partial.  n >= 0.
 */
int tp_shard_reduce(const float* const* Z_parts, int k, float* Z, int64_t n, void* stream);

/*
 * Bytes of device workspace tp_mlp_shard_forward needs: room for one Y_i
 * [M, Fk] (reused by every shard), plus k - 1 fp32 partials [M, H] unless
 * TP_FUSED_ACCUM is set (partial 0 is written into Z).  Returns 0 for invalid
 * arguments or M == 0.
 */
size_t tp_mlp_workspace_bytes(int k, int64_t M, int64_t H, int64_t Fk, int dtype, unsigned flags);

/*
 * The whole block forward over k shards, back to back on `stream`:
 *
 *   for i in 0..k-1:  Y = GeLU(X W[i] + b[i]);  P_i = Y V[i]
 *   Z = P_0 + P_1 + ... + P_{k-1}
 *
 * W, b and V are HOST arrays of k device pointers (b may be NULL for no bias;
 * otherwise every b[i] is non-NULL).  `workspace` is device memory of at least
 * tp_mlp_workspace_bytes(k, M, H, Fk, dtype, flags) bytes, 16-byte aligned.
 *
 * flags = 0: every P_i is materialised (P_0 in Z, the rest in the workspace)
 * and tp_shard_reduce sums them; this is the literal one-GPU stand-in for the
 * all-reduce.  flags = TP_FUSED_ACCUM: shard 0's row GEMM writes Z and shard
 * i > 0 adds its product into Z in its epilogue.  Both perform the same float32
 * additions in the same order and give bit-identical Z.
 */
int tp_mlp_shard_forward(const void* X, const void* const* W, const void* const* b,
                         const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                         int dtype, void* workspace, size_t workspace_bytes, float* Z,
                         unsigned flags, void* stream);

/* Static text for a status code. */
const char* tp_status_string(int status);

/* Library version, 100 * major + minor. */
int tp_mlp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H_ */
