// Internal launch interface between the C ABI (tp_mlp_abi.cpp) and the gfx950
// kernels.  Arguments are validated by the ABI layer before any of these is
// called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

// Epilogues of the tiled GEMM C[M,N] = A B, applied to the float32
// accumulator; "operand dtype" is bf16 for the bf16 GEMM, float32 for the
// float32 one.  aux is an [M, N] array with the leading dimension of C.
enum Epilogue : int {
  kEpiBiasGelu = 0,      // C = GeLU(acc + bias[n])                          (operand dtype)
  kEpiStoreF32 = 1,      // C = acc                                          (float32)
  kEpiAccumF32 = 2,      // C = C + acc                                      (float32)
  kEpiBiasGeluSave = 3,  // C = GeLU(acc + bias[n]), aux = GeLU'(acc + bias[n]) (operand dtype)
  kEpiMulAux = 4,        // C = acc * aux[m, n]; C may be aux itself         (operand dtype)
  kEpiSwiGLU = 5,        // C = SiLU(A B) * (A B2), two B operands (kNN)     (operand dtype)
  kEpiBias = 6,          // C = acc + bias[n]                                (operand dtype)
};

// Operand layouts.  A is logically [M, K] and B [K, N]:
//   kNN: A[m, k] at A[m * lda + k],  B[k, n] at B[k * ldb + n]
//   kNT: A[m, k] at A[m * lda + k],  B[k, n] at B[n * ldb + k]   (B stored transposed)
//   kTN: A[m, k] at A[k * lda + m],  B[k, n] at B[k * ldb + n]   (A stored transposed)
enum Layout : int { kNN = 0, kNT = 1, kTN = 2 };

struct GemmArgs {
  const void* A;
  const void* B;
  const void* bias;  // [N], kEpiBiasGelu / kEpiBiasGeluSave; may be null
  const void* B2;    // second B operand (same layout as B): kEpiSwiGLU
  void* C;           // [M, N], row m at C + m * ldc
  void* aux;         // [M, N] with leading dimension ldc: kEpiBiasGeluSave / kEpiMulAux
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  Layout layout;
  Epilogue epi;
};

// A batch of same-shaped GEMMs (the per-shard GEMMs of one step), launched
// together: group g computes C[g] = epi(A[g] B[g]) with bias[g] and aux[g]
// (entries may repeat, such as a shared X).  group_sum: instead, C[0] =
// sum_g A[g] B[g] with one float32 accumulator per group added in group
// order (kEpiAccumF32: C[0] + sum, in the same order), which is bit-identical
// to storing every product and summing them left to right.  kEpiSwiGLU
// groups also take a second B operand, B2[g].
constexpr int kMaxGroups = 16;
struct GemmBatch {
  const void* A[kMaxGroups];
  const void* B[kMaxGroups];
  const void* B2[kMaxGroups];
  const void* bias[kMaxGroups];
  void* C[kMaxGroups];
  void* aux[kMaxGroups];
  int groups;
  bool group_sum;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  Layout layout;
  Epilogue epi;
};

// bf16 operands (raw 16-bit patterns), float32 accumulate.  Requires the
// contiguous dimension of A, B and C to be a multiple of 8 elements, every
// leading dimension at most 2^22 elements, and 16-byte aligned pointers.
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_bf16_batch(const GemmBatch& b, hipStream_t s);

// The bf16 GEMM's tile table, for measuring the tile choice: the number of
// tiles; tile t's BM, BN, waves per workgroup and LDS stages; the tile a batch
// runs with; whether tile t is compiled for a batch's layout, epilogue, group
// sum and K; and the batch launched with tile t (every tile gives the same
// results, bit for bit: each output element is accumulated over K in the
// same order).
int gemm_bf16_tile_count();
void gemm_bf16_tile_shape(int tile, int info[4]);
int gemm_bf16_batch_tile(const GemmBatch& b);
bool gemm_bf16_tile_can_run(int tile, const GemmBatch& b);
hipError_t launch_gemm_bf16_batch_tile(int tile, const GemmBatch& b, hipStream_t s);

// float32 operands, float32 accumulate (same rules).  Batches run group by
// group (a group sum accumulates into C[0] in group order).
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_f32_batch(const GemmBatch& b, hipStream_t s);

// K-split of the GEMMs of a batch with a float32 output (kEpiStoreF32 /
// kEpiAccumF32) whose output has too few tiles to fill the chip (the weight
// gradients, where K is the token count): slice 0 writes (or adds into)
// C[g], slices 1..S-1 write float32 partials into `ws`, and each group's
// slices are then added into C[g] in slice order, so the result does not
// depend on timing.  C[g] must be dense (ldc == N).
int gemm_k_slices(bool bf16, int64_t tiles, int64_t K);
size_t gemm_split_workspace_bytes(bool bf16, int groups, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_split(const GemmBatch& b, bool bf16, void* ws, hipStream_t s);

// Z[e] = sum_i parts[i][e], i = 0..k-1 in order; Z may equal parts[0].
hipError_t launch_shard_reduce(const float* const* parts, int k, float* Z, int64_t n,
                               hipStream_t s);

// out[g][n] (+)= sum_m A[g][m, n] for `groups` matrices A[g] [M, N] row-major
// (bf16 when `bf16`, else float32), N a multiple of 8, in one pass of two
// launches.  Deterministic: rows are summed in fixed blocks whose float32
// partials go to `partials` and are then added in a fixed order.
// `partials` holds groups * colsum_partials_floats(M, N) floats.
int64_t colsum_partials_floats(int64_t M, int64_t N);
hipError_t launch_colsum(const void* const* A, int groups, bool bf16, int64_t M, int64_t N,
                         float* const* out, bool accumulate, float* partials, hipStream_t s);

// C[g][e] = C[g][e] + part[g (n-1)][e] + ... + part[g (n-1) + n-2][e] for
// 0 <= e < count and every group, in slice order (the K-split sums); part
// entries are part_stride floats apart.
hipError_t launch_split_reduce(float* const* C, int groups, const float* part, int64_t part_stride,
                               int n, int64_t count, hipStream_t s);

// Sequence-parallel reduce-scatter with the residual: for r < k,
// out[r][e] = R[r block_elems + e] + sum_i parts[i][r block_elems + e]
// (parts in order, then R; R may be null), 0 <= e < block_elems (a multiple
// of 8).  R is bf16 when r_bf16 (else float32); out[r] bf16 when o_bf16.
hipError_t launch_sp_reduce_scatter(const float* const* parts, int nparts, const void* R, bool r_bf16,
                                    void* const* out, bool o_bf16, int k, int64_t block_elems,
                                    hipStream_t s);

// dst[g] [C, R] = src[g]^T for row-major bf16 src[g] [R, C], g < groups;
// R and C multiples of 8, 16-byte aligned pointers.
hipError_t launch_transpose_bf16(const void* const* src, void* const* dst, int groups, int64_t R, int64_t C,
                                 hipStream_t s);

// Scaled dot-product attention of `heads` heads of dimension d (64 or 128)
// for `groups` shards at once: qkv[g] [B S, 3 heads d] bf16 (query, key and
// value of head h at columns h d, heads d + h d, 2 heads d + h d), out[g]
// [B S, heads d] bf16; causal masks keys after the query.  S <= 2^31 / (6
// heads d) keeps a sequence's rows within 32-bit offsets.
hipError_t launch_attention_bf16(const void* const* qkv, void* const* out, int groups, int64_t B,
                                 int64_t S, int heads, int d, bool causal, hipStream_t s);
// The same with a chosen kernel: 0 one query group of 32 per wave (128
// queries per workgroup), 1 two groups per wave (256 queries); -1 the
// library's choice.
hipError_t launch_attention_bf16_variant(int variant, const void* const* qkv, void* const* out, int groups,
                                         int64_t B, int64_t S, int heads, int d, bool causal, hipStream_t s);

// This device's copy of the static scratch array of the entry point that
// allocates nothing (TP_NOALLOC_SCRATCH_BYTES; the device of `stream`).
hipError_t noalloc_scratch(hipStream_t stream, void** out);

}  // namespace tpmlp
