/*
 * tp_mlp_dev.h — measurement hooks of libtpmlp.so (not part of the product
 * interface in tp_mlp.h): the tile table of the bf16 GEMM and entry points
 * that run a step with a tile of the caller's choice.  They exist to measure
 * the library's tile choice (which tile is fastest for each step and shape)
 * and to test that every tile gives the same result; a caller of the MLP
 * block has no need for them.  Types, status codes and flags are those of
 * tp_mlp.h.
 */
#ifndef TP_MLP_DEV_H_
#define TP_MLP_DEV_H_

#include "tp_mlp.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Tile table of the bf16 GEMM, for measuring the tile choice.  The bf16
 * column step (tp_mlp_col_gelu_shards without G: ColumnParallelLinear with
 * its bias and the GeLU, "AI大模型分布式训练：张量并行与流水线并行深度实践" §2.1)
 * and the row step (tp_mlp_row_partial_shards: RowParallelLinear's partial
 * products, §2.2 of the same page, and with TP_SUM_SHARDS their all-reduce
 * sum) run on a GEMM kernel compiled for a fixed table of output tiles; the
 * library picks one tile per launch from the shapes.  These calls
 * expose the table and run a step with a tile of the caller's choice.  Every
 * tile gives the same results, bit for bit (each output element is
 * accumulated over K in the same order); only the speed differs.
 */

/* Number of tiles in the table.  For 0 <= tile < count and info != NULL,
 * info[0..3] = BM, BN (output rows and columns of a workgroup), waves per
 * workgroup, LDS pipeline stages. */
int tp_gemm_tiles(int tile, int* info);

/* The tile the bf16 step runs with for n shards (1 <= n <= TP_MAX_BATCH) of
 * M tokens, width H and shard width Fk: step 0 = tp_mlp_col_gelu_shards
 * (G == NULL), 1 = tp_mlp_row_partial_shards, 2 = the same with
 * TP_SUM_SHARDS.  A negative status on invalid arguments. */
int tp_mlp_step_tile(int step, int n, int64_t M, int64_t H, int64_t Fk);

/* tp_mlp_col_gelu_shards (bf16, no G) with tile `tile`: the same arguments
 * and rules; TP_ERR_SHAPE if that tile is not compiled for this step (for
 * example K = H not a multiple of 32 on any tile but the ragged-K one). */
int tp_mlp_col_gelu_shards_tile(int tile, const void* X, const void* const* W, const void* const* b,
                                void* const* Y, int n, int64_t M, int64_t H, int64_t Fk, void* stream);

/* tp_mlp_row_partial_shards (bf16) with tile `tile`, as above (with
 * TP_SUM_SHARDS too). */
int tp_mlp_row_partial_shards_tile(int tile, const void* const* Y, const void* const* V, float* const* Z,
                                   int n, int64_t M, int64_t Fk, int64_t H, unsigned flags, void* stream);

/*
 * tp_attn_core_shards with a chosen attention kernel, for measuring the
 * library's choice between them (all give the same results, bit for bit;
 * the head-split attention of "AI大模型分布式训练：张量并行与流水线并行深度实践"
 * §2.3): variant 0 = one group of 32 queries per wave (4 waves, 128 queries
 * per workgroup), 1 = two groups per wave (256 queries per workgroup).  Other
 * arguments and rules as tp_attn_core_shards; TP_ERR_SHAPE for another
 * variant.
 */
int tp_attn_core_shards_variant(int variant, const void* const* QKV, void* const* A, int n, int64_t B, int64_t S,
                                int heads, int head_dim, int dtype, unsigned flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_DEV_H_ */
