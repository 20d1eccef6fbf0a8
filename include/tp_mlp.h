/*
 * tp_mlp.h — C ABI of libtpmlp.so: the forward and backward passes of one
 * Megatron-style tensor-parallel MLP block, every shard of it on one AMD
 * Instinct MI355X (gfx950).
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
 * Constraints.  H and Fk are multiples of 8, at least 8 and at most 2^22
 * (the kernels address the rows of a tile with 32-bit offsets); M >= 0 (for
 * the forward entry points M == 0 is a no-op that returns TP_OK);
 * 1 <= k <= TP_MAX_SHARDS; M < 2^31 and each matrix holds fewer than 2^40
 * elements; every pointer is 16-byte aligned.  Outputs must not overlap
 * inputs or each other unless stated.
 *
 * Backward.  The entry points after tp_mlp_shard_forward compute the
 * gradients of the same block for a loss L, given dZ = dL/dZ.  In the
 * tensor-parallel block the forward all-reduce becomes an identity in the
 * backward pass and the (identity) broadcast of X becomes an all-reduce of
 * the input gradient, so every shard sees the same dZ, computes its own
 * parameter gradients and a partial dX_i, and the partials are summed
 * ("大模型分布式训练四维并行：DDP、ZeRO、张量、流水线与上下文" §4.3: the backward
 * exchange mirrors the forward one; "AI大模型分布式训练：张量并行与流水线并行深度实践"
 * §2.4: forward and backward each take one all-reduce per MLP):
 *
 *     A_i  = X W_i + b_i,  G_i = GeLU'(A_i) = Phi(A_i) + A_i phi(A_i)
 *     dA_i = (dZ V_i^T) * G_i             (element-wise product)
 *     dV_i = Y_i^T dZ,  dW_i = X^T dA_i,  db_i = sum over rows of dA_i
 *     dX_i = dA_i W_i^T,  dX = dX_0 + ... + dX_{k-1}
 *
 * with phi the standard normal density.  dZ [M, H] has the input dtype;
 * G_i and dA_i [M, Fk] have the input dtype; dV_i [Fk, H], dW_i [H, Fk],
 * db_i [Fk], dX_i and dX [M, H] are float32.  In TP_BF16 the products
 * accumulate in float32 and G_i, dA_i are rounded to bfloat16 once.
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
#define TP_MAX_BATCH 16 /* shards per call of the *_shards entry points */

/* Flags. */
#define TP_ACCUMULATE 1u  /* tp_mlp_row_partial, tp_mlp_grad_input_partial: add into the output */
#define TP_FUSED_ACCUM 1u /* tp_mlp_shard_forward / _backward: fold the shard sum into the GEMMs */
#define TP_GRAD_ACCUMULATE 2u /* weight-gradient entry points: add into dW, db, dV */
#define TP_SUM_SHARDS 4u      /* row / input-gradient batches: one output, the shard-order sum */
#define TP_CAUSAL 8u          /* attention: each query attends to keys at or before it only */

/* Size of the device scratch array of tp_mlp_shard_forward_noalloc (per GPU). */
#define TP_NOALLOC_SCRATCH_BYTES (128u << 20)

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
 * Bytes of device workspace tp_mlp_shard_forward needs: one Y_i [M, Fk] per
 * shard of a batch (the shards run in batches of up to 16, each step of a
 * batch in one launch), plus k - 1 fp32 partials [M, H] unless
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
 * all-reduce.  flags = TP_FUSED_ACCUM: the row GEMMs of a batch of shards run
 * as one kernel in which every output tile carries one float32 accumulator
 * through the products of every shard in shard order, so no partial goes
 * through memory: the row-parallel identity sum_i Y_i V_i = [Y_0 ... Y_{k-1}] V
 * ("千亿参数模型如何拆分到多张GPU上训练", 方案二) evaluated as the unsplit GEMM.
 * The two variants give the same sum up to float32 rounding; each is
 * deterministic (the same bits on every run).
 */
int tp_mlp_shard_forward(const void* X, const void* const* W, const void* const* b,
                         const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                         int dtype, void* workspace, size_t workspace_bytes, float* Z,
                         unsigned flags, void* stream);

/*
 * tp_mlp_shard_forward without a workspace argument and without any memory
 * allocation, for callers that cannot allocate device memory during the call:
 * code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, results and errors are those of
 * tp_mlp_shard_forward (the same Z, bit for bit, for the same flags); the
 * intermediate Y_i and, for the literal variant, the k - 1 float32 partials
 * live in a static device array of TP_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.  The shards run in
 * batches small enough for the array; when even one shard's Y_i [M, Fk]
 * (plus, literal, the k - 1 partials [M, H] of 4 bytes) does not fit, the
 * call returns TP_ERR_WORKSPACE before any launch.  It calls no hipMalloc or
 * hipFree; the first call on a GPU places the array there (the HIP runtime
 * loads the library code that holds it), so make one call before capturing
 * a graph.  All calls on one GPU share its array: calls that overlap in time
 * on one GPU (on different streams, or from different threads) race on it
 * and must be ordered by the caller.  The device is that of `stream`.
 */
int tp_mlp_shard_forward_noalloc(const void* X, const void* const* W, const void* const* b,
                                 const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                                 int dtype, float* Z, unsigned flags, void* stream);

/*
 * Sequence parallelism.  Megatron's sequence parallelism also splits the
 * part of the block that tensor parallelism leaves whole (LayerNorm,
 * Dropout, the residual) along the sequence, one block of M/k rows per rank
 * ("AI大模型分布式训练：张量并行与流水线并行深度实践" §4.2; "大模型分布式训练四维并行：
 * DDP、ZeRO、张量、流水线与上下文" §4.3).  The all-reduce that ends the
 * row-parallel layer is then cut at its midpoint: an all-reduce is a
 * reduce-scatter followed by an all-gather (the ring algorithm, §2.1 of the
 * latter page), and each rank keeps only its reduce-scatter block.  The
 * block's residual connection x + mlp(x) (the TransformerBlock of §3.4 of the
 * former page) is added to that block in the same pass:
 *
 *   for r in 0..k-1, m in 0..M/k-1:
 *     O[r][m, n] = R[r M/k + m, n] + (Z_parts[0] + ... + Z_parts[nparts-1])[r M/k + m, n]
 *
 * The parts are float32 [M, H] and are summed left to right in float32, then
 * R is added (R == NULL: no residual) and the result is stored in
 * `out_dtype` (rounded to nearest-even for TP_BF16).  R [M, H] has type
 * `r_dtype`.  Z_parts is a HOST array of nparts device pointers
 * (1 <= nparts <= TP_MAX_SHARDS) and O a HOST array of k device pointers to
 * [M/k, H] blocks (1 <= k <= TP_MAX_SHARDS, k divides M).  Passing
 * O[r] = base + r (M/k) H elements puts the blocks side by side, which is
 * the all-gather on one device.  H follows the rules above; M == 0 is a
 * no-op.  No output may overlap an input or another output.
 */
int tp_sp_reduce_scatter(const float* const* Z_parts, int nparts, const void* R, int r_dtype,
                         void* const* O, int out_dtype, int k, int64_t M, int64_t H, void* stream);

/*
 * Bytes of device workspace tp_mlp_shard_forward_sp needs: one Y_i per shard
 * of a batch (as tp_mlp_workspace_bytes) plus k float32 partials [M, H], or
 * one (their running sum) with TP_FUSED_ACCUM.  0 for invalid arguments,
 * M == 0 or k not dividing M.
 */
size_t tp_mlp_sp_workspace_bytes(int k, int64_t M, int64_t H, int64_t Fk, int dtype, unsigned flags);

/*
 * The block forward under sequence parallelism: tp_mlp_shard_forward whose
 * closing all-reduce is tp_sp_reduce_scatter with X as the residual,
 *
 *   O[r] = X[rows of r] + (P_0 + ... + P_{k-1})[rows of r],  P_i = GeLU(X W[i] + b[i]) V[i]
 *
 * (on one device the all-gather of X that precedes the column-parallel layer
 * under sequence parallelism is X itself).  Arguments as for
 * tp_mlp_shard_forward, with O a HOST array of k device pointers to [M/k, H]
 * blocks of `out_dtype`, which k must divide M, and `workspace` of
 * tp_mlp_sp_workspace_bytes(...) bytes.  flags = TP_FUSED_ACCUM sums the
 * shards inside the row GEMMs (one partial in memory instead of k), as for
 * tp_mlp_shard_forward; the float32 blocks equal X + Z of
 * tp_mlp_shard_forward with the same flags, bit for bit.
 */
int tp_mlp_shard_forward_sp(const void* X, const void* const* W, const void* const* b,
                            const void* const* V, int k, int64_t M, int64_t H, int64_t Fk,
                            int dtype, void* workspace, size_t workspace_bytes, void* const* O,
                            int out_dtype, unsigned flags, void* stream);

/*
 * SwiGLU variant of the block (the gated MLP of Llama-style models: gate_proj
 * and up_proj column-parallel, down_proj row-parallel, "AI大模型分布式训练：张量
 * 并行与流水线并行深度实践" §6.1; gate_up_proj column- and down_proj
 * row-parallel, "大模型分布式优化技术（一）" §5.1).  The pages name the SwiGLU
 * activation (§3.3 of the latter) without its formula; it is taken here as
 * Llama's, without biases:
 *
 *   Y_i = SiLU(X Wg_i) * (X Wu_i),  SiLU(x) = x / (1 + exp(-x))
 *   Z_i = Y_i V_i,  Z = Z_0 + ... + Z_{k-1}
 *
 * Wg_i and Wu_i [H, Fk] are columns [i*Fk, (i+1)*Fk) of the full gate and up
 * weights [H, F] (type `dtype`, row-major [in, out]); both products of a tile
 * run in one GEMM and the activation is applied to the two float32
 * accumulators before Y_i is rounded to `dtype`.  The row step and the shard
 * sum are those of the GeLU block.
 *
 * tp_swiglu_col: one shard's column step, Y_i [M, Fk] must not overlap X,
 * Wg_i or Wu_i.  tp_swiglu_col_shards: the same for n shards in one launch
 * (as the other *_shards calls).  tp_swiglu_shard_forward: the whole block,
 * arguments and flags as tp_mlp_shard_forward (Wg, Wu, V HOST arrays of k
 * device pointers; workspace of tp_mlp_workspace_bytes(k, M, H, Fk, dtype,
 * flags) bytes).
 */
int tp_swiglu_col(const void* X, const void* Wg_i, const void* Wu_i, void* Y_i, int64_t M, int64_t H,
                  int64_t Fk, int dtype, void* stream);
int tp_swiglu_col_shards(const void* X, const void* const* Wg, const void* const* Wu, void* const* Y,
                         int n, int64_t M, int64_t H, int64_t Fk, int dtype, void* stream);
int tp_swiglu_shard_forward(const void* X, const void* const* Wg, const void* const* Wu,
                            const void* const* V, int k, int64_t M, int64_t H, int64_t Fk, int dtype,
                            void* workspace, size_t workspace_bytes, float* Z, unsigned flags,
                            void* stream);

/*
 * Tensor-parallel attention block (multi-head attention split by heads: each
 * of the k shards owns n_heads / k whole heads, its Q/K/V projection is
 * column-parallel, its heads' attention needs no communication, and the
 * output projection is row-parallel and summed: "AI大模型分布式训练：张量并行与流水线
 * 并行深度实践" §2.3; "千亿参数模型如何拆分到多张GPU上训练" 注意力层的切分;
 * "大模型分布式并行策略详解：TP、DP、PP、CP、EP核心原理与实战" §4.2).  With
 * d = H / n_heads (64 or 128), hk = n_heads / k and Hk = hk d, for rows
 * m = b S + t of X [B S, H]:
 *
 *   QKV_i = X Wqkv_i + bqkv_i                [M, 3 Hk]: q | k | v of shard i
 *   per head h of the shard, within each sequence:
 *     o_t = sum_j softmax_j(q_t . k_j / sqrt(d)) v_j   (j <= t with TP_CAUSAL)
 *   A_i = the heads' outputs side by side    [M, Hk]
 *   Z_i = A_i Wo_i,  Z = Z_0 + ... + Z_{k-1}  (Wo_i [Hk, H], rows block i of Wo)
 *
 * Wqkv_i [H, 3 Hk] holds the columns of shard i's heads of the full Wq, Wk and
 * Wv side by side ([Wq_i | Wk_i | Wv_i], the layout of one
 * ColumnParallelLinear(H, 3H) shard whose output is chunked into q, k, v);
 * bqkv_i [3 Hk] likewise (NULL: no bias).  TP_BF16 only for the attention
 * (TP_ERR_DTYPE otherwise): the projection accumulates in float32 and is
 * rounded to bf16, the scores, softmax and weighted sum are float32 (the
 * probabilities rounded to bf16 for the products with V), A_i is rounded to
 * bf16, Z is float32.
 *
 * tp_attn_qkv_shards: the projection for n shards (any dtype; 3 Hk <= 2^22).
 * tp_attn_core_shards: each shard's attention, QKV[i] [B S, 3 heads d] ->
 * A[i] [B S, heads d], flags = TP_CAUSAL or 0.  tp_attn_shard_forward: the
 * block, workspace of tp_attn_workspace_bytes(...) bytes, flags
 * TP_FUSED_ACCUM (the output projections sum the shards inside the GEMM, as
 * for the MLP) and TP_CAUSAL.  M == 0 is a no-op; S * 6 Hk < 2^31.
 */
int tp_attn_qkv_shards(const void* X, const void* const* Wqkv, const void* const* bqkv, void* const* QKV,
                       int n, int64_t M, int64_t H, int64_t Hk, int dtype, void* stream);
int tp_attn_core_shards(const void* const* QKV, void* const* A, int n, int64_t B, int64_t S, int heads,
                        int head_dim, int dtype, unsigned flags, void* stream);
size_t tp_attn_workspace_bytes(int k, int64_t B, int64_t S, int64_t H, int n_heads, int dtype,
                               unsigned flags);
int tp_attn_shard_forward(const void* X, const void* const* Wqkv, const void* const* bqkv,
                          const void* const* Wo, int k, int64_t B, int64_t S, int64_t H, int n_heads,
                          int dtype, void* workspace, size_t workspace_bytes, float* Z, unsigned flags,
                          void* stream);

/*
 * Training-mode column step: tp_mlp_col_gelu that also keeps the derivative
 * of the activation for the backward pass (the closed form of GeLU' above):
 *
 *   Y_i[m, j] = GeLU(A_i[m, j]),  G_i[m, j] = GeLU'(A_i[m, j]),
 *   A_i = X W_i + b_i
 *
 * Same arguments as tp_mlp_col_gelu plus G_i [M, Fk] of type `dtype`, which
 * must not overlap any other argument.
 */
int tp_mlp_col_gelu_save(const void* X, const void* W_i, const void* b_i, void* Y_i, void* G_i,
                         int64_t M, int64_t H, int64_t Fk, int dtype, void* stream);

/*
 * Gradient at the pre-activation of shard i (the backward of the row-parallel
 * linear through the activation):
 *
 *   dA_i[m, j] = G_i[m, j] * sum_n dZ[m, n] V_i[j, n]
 *
 * dZ [M, H], V_i [Fk, H], G_i and dA_i [M, Fk], all of type `dtype`.  dA_i may
 * be G_i itself (in place); otherwise it must not overlap any input.
 */
int tp_mlp_grad_act(const void* dZ, const void* V_i, const void* G_i, void* dA_i, int64_t M,
                    int64_t H, int64_t Fk, int dtype, void* stream);

/*
 * Bytes of device workspace that tp_mlp_grad_row_weight and
 * tp_mlp_grad_col_weight need for these sizes (room for the partial products
 * of a K-split of the M rows and for the column-sum partials of db_i).
 * Returns 0 for invalid arguments.
 */
size_t tp_mlp_grad_weight_workspace_bytes(int64_t M, int64_t H, int64_t Fk, int dtype);

/*
 * Weight gradient of the row-parallel linear of shard i:
 *
 *   dV_i[j, n] = sum_m Y_i[m, j] dZ[m, n]               (flags = 0)
 *   dV_i[j, n] = dV_i[j, n] + sum_m Y_i[m, j] dZ[m, n]  (TP_GRAD_ACCUMULATE)
 *
 * Y_i [M, Fk], dZ [M, H] of type `dtype`; dV_i [Fk, H] float32.  M == 0 gives
 * zeros (or leaves dV_i unchanged with TP_GRAD_ACCUMULATE); Y_i and dZ may
 * then be NULL.  `workspace`:
 * device memory of tp_mlp_grad_weight_workspace_bytes(M, H, Fk, dtype) bytes
 * (may be NULL when that is 0).  Sums over m are formed in float32 in a fixed
 * order, so the result is deterministic.
 */
int tp_mlp_grad_row_weight(const void* Y_i, const void* dZ, float* dV_i, int64_t M, int64_t Fk,
                           int64_t H, int dtype, void* workspace, size_t workspace_bytes,
                           unsigned flags, void* stream);

/*
 * Weight and bias gradients of the column-parallel linear of shard i:
 *
 *   dW_i[h, j] = sum_m X[m, h] dA_i[m, j],   db_i[j] = sum_m dA_i[m, j]
 *
 * X [M, H], dA_i [M, Fk] of type `dtype`; dW_i [H, Fk] and db_i [Fk] float32
 * (db_i may be NULL: no bias gradient).  TP_GRAD_ACCUMULATE adds into dW_i
 * and db_i.  Workspace, M == 0 and determinism as for tp_mlp_grad_row_weight.
 */
int tp_mlp_grad_col_weight(const void* X, const void* dA_i, float* dW_i, float* db_i, int64_t M,
                           int64_t H, int64_t Fk, int dtype, void* workspace,
                           size_t workspace_bytes, unsigned flags, void* stream);

/*
 * Partial input gradient of shard i, the term the backward all-reduce sums:
 *
 *   dX_i[m, h] = sum_j dA_i[m, j] W_i[h, j]          (flags = 0)
 *   dX_i[m, h] = dX_i[m, h] + sum_j ...             (TP_ACCUMULATE)
 *
 * dA_i [M, Fk], W_i [H, Fk] of type `dtype`; dX_i [M, H] float32.
 */
int tp_mlp_grad_input_partial(const void* dA_i, const void* W_i, float* dX_i, int64_t M,
                              int64_t Fk, int64_t H, int dtype, unsigned flags, void* stream);

/*
 * Bytes of device workspace tp_mlp_shard_backward needs: Y_i and G_i / dA_i
 * [M, Fk] for every shard of a batch (up to 16), the weight-gradient
 * workspace of a batch, k - 1 float32 partials [M, H] unless TP_FUSED_ACCUM
 * is set, and for bf16 with M >= 4096 transposed copies of W_i and V_i
 * (bf16 [Fk, H] and [H, Fk]) for every shard of a batch, through which the
 * products by W_i^T and V_i^T run.  Returns 0 for invalid arguments.
 */
size_t tp_mlp_backward_workspace_bytes(int k, int64_t M, int64_t H, int64_t Fk, int dtype,
                                       unsigned flags);

/*
 * The whole block backward over k shards, back to back on `stream`; Y_i and
 * G_i are recomputed from X (activation recomputation), so nothing from the
 * forward call needs to be kept:
 *
 *   for i in 0..k-1:
 *     Y, G = GeLU(A_i), GeLU'(A_i)          tp_mlp_col_gelu_save
 *     dA   = (dZ V[i]^T) * G               tp_mlp_grad_act (in place over G)
 *     dV[i] = Y^T dZ                        tp_mlp_grad_row_weight
 *     dW[i] = X^T dA,  db[i] = colsum(dA)   tp_mlp_grad_col_weight
 *     P_i  = dA W[i]^T                      tp_mlp_grad_input_partial
 *   dX = P_0 + P_1 + ... + P_{k-1}          tp_shard_reduce
 *
 * W, b, V, dW, db and dV are HOST arrays of k device pointers (b == NULL: no
 * bias; db == NULL: no bias gradient; otherwise every entry is non-NULL).
 * flags: TP_FUSED_ACCUM folds the sum of the P_i into the dX GEMMs (one
 * float32 accumulator through every shard's products, as in the forward; the
 * same dX up to float32 rounding);
 * TP_GRAD_ACCUMULATE adds into dW, db and dV.  M == 0 leaves dX empty and
 * gives zero (or unchanged) parameter gradients; X, dZ and dX may then be
 * NULL.
 */
int tp_mlp_shard_backward(const void* X, const void* const* W, const void* const* b,
                          const void* const* V, const void* dZ, int k, int64_t M, int64_t H,
                          int64_t Fk, int dtype, void* workspace, size_t workspace_bytes,
                          float* dX, float* const* dW, float* const* db, float* const* dV,
                          unsigned flags, void* stream);

/*
 * Batched steps.  Each *_shards call runs one step for n shards
 * (1 <= n <= TP_MAX_BATCH) of the same shapes as one launch, so that the
 * small per-shard GEMMs of a narrow layer fill the chip; it gives the same
 * results, bit for bit, as n calls of the single-shard entry point.  Array
 * arguments are HOST arrays of n device pointers; every rule of the
 * single-shard call applies to each shard, and no output may overlap an
 * input or another output.
 */

/* tp_mlp_col_gelu (G == NULL) or tp_mlp_col_gelu_save for shards 0..n-1:
 * X shared; W[i], b[i] (b == NULL: no bias), Y[i] and G[i] per shard. */
int tp_mlp_col_gelu_shards(const void* X, const void* const* W, const void* const* b, void* const* Y,
                           void* const* G, int n, int64_t M, int64_t H, int64_t Fk, int dtype,
                           void* stream);

/* tp_mlp_row_partial for shards 0..n-1: Z[i] (+)= Y[i] V[i].  With
 * TP_SUM_SHARDS, Z[0] = Y[0] V[0] + ... + Y[n-1] V[n-1] (or Z[0] + ... with
 * TP_ACCUMULATE) as one GEMM [Y[0] ... Y[n-1]] [V[0]; ...; V[n-1]]: one float32
 * accumulator per output element runs through the shards in order (starting
 * at Z[0] with TP_ACCUMULATE, so a batch split over several calls gives the
 * same bits as one call); equal to n partials followed by tp_shard_reduce up
 * to float32 rounding (only Z[0] is used). */
int tp_mlp_row_partial_shards(const void* const* Y, const void* const* V, float* const* Z, int n,
                              int64_t M, int64_t Fk, int64_t H, int dtype, unsigned flags,
                              void* stream);

/* tp_mlp_grad_act for shards 0..n-1 (dZ shared; dA[i] may be G[i]). */
int tp_mlp_grad_act_shards(const void* dZ, const void* const* V, const void* const* G,
                           void* const* dA, int n, int64_t M, int64_t H, int64_t Fk, int dtype,
                           void* stream);

/* Workspace of tp_mlp_grad_row_weight_shards / tp_mlp_grad_col_weight_shards
 * for n shards (n == 1: tp_mlp_grad_weight_workspace_bytes).  0 on invalid
 * arguments. */
size_t tp_mlp_grad_weight_workspace_bytes_shards(int n, int64_t M, int64_t H, int64_t Fk,
                                                 int dtype);

/* tp_mlp_grad_row_weight for shards 0..n-1 (dZ shared). */
int tp_mlp_grad_row_weight_shards(const void* const* Y, const void* dZ, float* const* dV, int n,
                                  int64_t M, int64_t Fk, int64_t H, int dtype, void* workspace,
                                  size_t workspace_bytes, unsigned flags, void* stream);

/* tp_mlp_grad_col_weight for shards 0..n-1 (X shared; db == NULL: no bias
 * gradients). */
int tp_mlp_grad_col_weight_shards(const void* X, const void* const* dA, float* const* dW,
                                  float* const* db, int n, int64_t M, int64_t H, int64_t Fk,
                                  int dtype, void* workspace, size_t workspace_bytes,
                                  unsigned flags, void* stream);

/* tp_mlp_grad_input_partial for shards 0..n-1; TP_SUM_SHARDS as for
 * tp_mlp_row_partial_shards (the backward all-reduce of dX folded in). */
int tp_mlp_grad_input_shards(const void* const* dA, const void* const* W, float* const* dX, int n,
                             int64_t M, int64_t Fk, int64_t H, int dtype, unsigned flags,
                             void* stream);

/* Static text for a status code. */
const char* tp_status_string(int status);

/* Library version, 100 * major + minor. */
int tp_mlp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H_ */
