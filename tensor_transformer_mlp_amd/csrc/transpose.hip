// Batched bf16 matrix transpose for gfx950: dst[g] [C, R] = src[g]^T for
// row-major src[g] [R, C].  The backward pass uses it to turn the weights it
// multiplies by their transposes (dZ V_i^T and dA_i W_i^T) into N-major
// operands, so that those products run on the GEMM's NN path.
#include "device_common.h"
#include "tp_mlp_kernels.h"

namespace tpmlp {

namespace {

struct TransposePtrs {
  const uint16_t* src[kMaxGroups];
  uint16_t* dst[kMaxGroups];
};

constexpr int kT = 64;           // tile edge (elements)
constexpr int kTPitch = kT + 2;  // LDS row pitch (elements): spreads a column over the banks

// One 64 x 64 tile per workgroup: 16-byte loads along src rows into LDS, then
// 16-byte stores along dst rows (8 consecutive src rows of one src column).
// R and C are multiples of 8, so every 8-element chunk is wholly inside or
// wholly outside the matrix.
// Grid: x = tile index (column tiles fastest), y = group.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(TransposePtrs t, int64_t R, int64_t C) {
  __shared__ uint16_t tile[kT * kTPitch];
  const int g = blockIdx.y;
  const int64_t ct = (C + kT - 1) / kT;
  const int64_t c0 = ((int64_t)blockIdx.x % ct) * kT, r0 = ((int64_t)blockIdx.x / ct) * kT;
  const uint16_t* src = t.src[g];
  uint16_t* dst = t.dst[g];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = threadIdx.x + 256 * h;  // 512 chunks: 64 rows x 8
    const int row = idx >> 3, ch = idx & 7;
    const int64_t r = r0 + row, c = c0 + 8 * ch;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (r < R && c < C) v = *reinterpret_cast<const u32x4_t*>(src + r * C + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[row * kTPitch + 8 * ch + 2 * i] = (uint16_t)(v[i] & 0xFFFFu);
      tile[row * kTPitch + 8 * ch + 2 * i + 1] = (uint16_t)(v[i] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int idx = threadIdx.x + 256 * h;  // 512 chunks: 64 dst rows x 8
    const int orow = idx >> 3, ch = idx & 7;
    const int64_t c = c0 + orow, r = r0 + 8 * ch;
    if (c >= C || r >= R) continue;
    u32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (uint32_t)tile[(8 * ch + 2 * i) * kTPitch + orow] |
             ((uint32_t)tile[(8 * ch + 2 * i + 1) * kTPitch + orow] << 16);
    *reinterpret_cast<u32x4_t*>(dst + c * R + r) = v;
  }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* const* src, void* const* dst, int groups, int64_t R, int64_t C,
                                 hipStream_t s) {
  if (groups < 1 || groups > kMaxGroups || R % 8 || C % 8) return hipErrorInvalidValue;
  if (R <= 0 || C <= 0) return hipSuccess;
  TransposePtrs t{};
  for (int g = 0; g < groups; ++g) {
    t.src[g] = static_cast<const uint16_t*>(src[g]);
    t.dst[g] = static_cast<uint16_t*>(dst[g]);
  }
  // one dimension for the tiles: a matrix of fewer than 2^40 elements has
  // fewer than 2^28 of them (the y and z grid dimensions stop at 65535)
  const int64_t tiles = ((C + kT - 1) / kT) * ((R + kT - 1) / kT);
  if (tiles >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tiles, (unsigned)groups);
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, t, R, C);
  return hipGetLastError();
}

}  // namespace tpmlp
