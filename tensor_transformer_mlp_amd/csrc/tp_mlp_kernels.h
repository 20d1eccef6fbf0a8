// Internal launch interface between the C ABI (tp_mlp_abi.cpp) and the gfx950
// kernels (tp_mlp_kernels.hip).  Arguments are validated by the ABI layer
// before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

// Epilogues of the tiled GEMM C[M,N] = A[M,K] B[K,N].
enum Epilogue : int {
  kEpiBiasGelu = 0,  // C = GeLU(acc + bias[n]) in the input dtype
  kEpiStoreF32 = 1,  // C = acc (float32)
  kEpiAccumF32 = 2,  // C = C + acc (float32)
};

// bf16 operands (raw 16-bit patterns), float32 accumulate.
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, const uint16_t* bias, void* C,
                            int64_t M, int64_t N, int64_t K, Epilogue epi, hipStream_t s);

// float32 operands, float32 accumulate.
hipError_t launch_gemm_f32(const float* A, const float* B, const float* bias, void* C, int64_t M,
                           int64_t N, int64_t K, Epilogue epi, hipStream_t s);

// Z[e] = sum_i parts[i][e], i = 0..k-1 in order; Z may equal parts[0].
hipError_t launch_shard_reduce(const float* const* parts, int k, float* Z, int64_t n,
                               hipStream_t s);

}  // namespace tpmlp
