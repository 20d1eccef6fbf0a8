// Streaming reductions for gfx950: the sum of the k shard partials (the
// one-device stand-in for the all-reduce) and a deterministic column sum.
#include "device_common.h"
#include "tp_mlp_kernels.h"

namespace tpmlp {

namespace {

// ---------------------------------------------------------------------------
// Shard reduce: Z = ((P_0 + P_1) + P_2) + ... in float32, 16-byte vectors,
// grid-stride.  KC > 0 fixes k at compile time so that all k loads of a
// vector are in flight together; KC == 0 reads k at run time.
// ---------------------------------------------------------------------------
struct PartPtrs {
  const float* p[64];
};

// U 16-byte vectors per thread per iteration, all 1 + (k - 1) loads of them
// issued before the adds, so that each thread keeps U * k loads in flight.
template <int KC, int U>
__global__ __launch_bounds__(256) void shard_reduce_kernel(PartPtrs parts, int k,
                                                           float* __restrict__ Z, int64_t n) {
  const int kk = KC > 0 ? KC : k;
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
  for (int64_t v0 = ((int64_t)blockIdx.x * blockDim.x) * U + threadIdx.x; v0 < n4; v0 += stride) {
    f32x4_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      s[u] = v < n4 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[0]) + v)
                    : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (KC > 0) {
      f32x4_t t[KC > 1 ? KC - 1 : 1][U];
#pragma unroll
      for (int i = 1; i < KC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          t[i - 1][u] = v < n4 ? __builtin_nontemporal_load(
                                     reinterpret_cast<const f32x4_t*>(parts.p[i]) + v)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int i = 1; i < KC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = s[u] + t[i - 1][u];
    } else {
      for (int i = 1; i < kk; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          if (v < n4)
            s[u] = s[u] + __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(parts.p[i]) + v);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      if (v < n4) __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4_t*>(Z) + v);
    }
  }
  // scalar tail (n not a multiple of 4)
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t e = (n4 << 2) + threadIdx.x;
    float s = parts.p[0][e];
    for (int i = 1; i < kk; ++i) s = s + parts.p[i][e];
    Z[e] = s;
  }
}

template <int U>
hipError_t launch_reduce_u(const PartPtrs& pp, int k, float* Z, int64_t n, int64_t max_blocks,
                           hipStream_t s) {
  const int64_t n4 = n >> 2;
  int64_t blocks = (n4 + 256 * U - 1) / (256 * U);
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks), block(256);
  switch (k) {
    case 1: hipLaunchKernelGGL((shard_reduce_kernel<1, U>), grid, block, 0, s, pp, k, Z, n); break;
    case 2: hipLaunchKernelGGL((shard_reduce_kernel<2, U>), grid, block, 0, s, pp, k, Z, n); break;
    case 4: hipLaunchKernelGGL((shard_reduce_kernel<4, U>), grid, block, 0, s, pp, k, Z, n); break;
    case 8: hipLaunchKernelGGL((shard_reduce_kernel<8, U>), grid, block, 0, s, pp, k, Z, n); break;
    default: hipLaunchKernelGGL((shard_reduce_kernel<0, U>), grid, block, 0, s, pp, k, Z, n); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Column sum out[n] (+)= sum_m A[m, n], two passes:
//   1. workgroup (cb, rb) sums rows [rb R, rb R + R) of columns
//      [256 cb, 256 cb + 256): 32 column groups of 8 x 8 row lanes, each lane
//      a running float32 sum over every 8th row, then the 8 row lanes are
//      added in order through LDS; the result is partials[rb][n];
//   2. out[n] = (out[n] +) the partials of column n, in a fixed order: four
//      consecutive runs of row blocks, each summed in order, then the four
//      run sums in order.
// The row-block count depends only on (M, N), so the result is reproducible.
// ---------------------------------------------------------------------------
constexpr int kColsPerBlock = 256;

int64_t colsum_row_blocks(int64_t M, int64_t N) {
  if (M <= 0) return 0;
  const int64_t cb = (N + kColsPerBlock - 1) / kColsPerBlock;
  int64_t rb = (2048 + cb - 1) / cb;        // aim for ~2048 workgroups
  const int64_t max_rb = (M + 63) / 64;      // at least 64 rows per workgroup
  if (rb > max_rb) rb = max_rb;
  if (rb > 4096) rb = 4096;
  return rb < 1 ? 1 : rb;
}

struct ColsumPtrs {
  const void* A[kMaxGroups];
  float* out[kMaxGroups];
};

// blockIdx.z: the group (shard) whose A is summed into partials + z rb N.
template <bool BF16>
__global__ __launch_bounds__(256) void colsum_partial_kernel(ColsumPtrs pp, int64_t M, int64_t N,
                                                             int64_t rows_per_block,
                                                             float* __restrict__ partials_all) {
  __shared__ float red[8][kColsPerBlock + 4];
  const void* __restrict__ A = pp.A[blockIdx.z];
  float* __restrict__ partials = partials_all + (int64_t)blockIdx.z * gridDim.y * N;
  const int cg = threadIdx.x & 31, rl = threadIdx.x >> 5;
  const int64_t n = (int64_t)blockIdx.x * kColsPerBlock + cg * 8;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  int64_t r1 = r0 + rows_per_block;
  if (r1 > M) r1 = M;
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.f;
  if (n < N) {
#pragma unroll 8
    for (int64_t r = r0 + rl; r < r1; r += 8) {
      if constexpr (BF16) {
        const u32x4_t v =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(A) + r * N + n));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[2 * e] += bf16_bits_to_f32(v[e] & 0xFFFFu);
          s[2 * e + 1] += bf16_bits_to_f32(v[e] >> 16);
        }
      } else {
        const f32x4_t* q = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(A) + r * N + n);
        const f32x4_t a = __builtin_nontemporal_load(q), b = __builtin_nontemporal_load(q + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[e] += a[e];
          s[4 + e] += b[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rl][cg * 8 + e] = s[e];
  __syncthreads();
  const int c = threadIdx.x;  // one column of the block per thread
  const int64_t nc = (int64_t)blockIdx.x * kColsPerBlock + c;
  if (nc < N) {
    float t = red[0][c];
#pragma unroll
    for (int i = 1; i < 8; ++i) t += red[i][c];
    partials[(int64_t)blockIdx.y * N + nc] = t;
  }
}

// Pass 2: 64 columns per workgroup, 4 row groups of 64 lanes; group g adds
// partial rows [g q, (g + 1) q) in order, and the four group sums are then
// added in group order (q = ceil(rb / 4)), so the order is fixed by (M, N).
__global__ __launch_bounds__(256) void colsum_final_kernel(ColsumPtrs pp, const float* __restrict__ partials_all,
                                                           int64_t rb, int64_t N, int accumulate) {
  __shared__ float red[4][64];
  const float* __restrict__ partials = partials_all + (int64_t)blockIdx.y * rb * N;
  float* __restrict__ out = pp.out[blockIdx.y];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + c;
  const int64_t q = (rb + 3) / 4;
  const int64_t i0 = g * q;
  const int64_t i1 = i0 + q < rb ? i0 + q : rb;
  float t = 0.f;
  if (n < N) {
    int64_t i = i0;
    for (; i + 8 <= i1; i += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = partials[(i + u) * N + n];
#pragma unroll
      for (int u = 0; u < 8; ++u) t += v[u];
    }
    for (; i < i1; ++i) t += partials[i * N + n];
  }
  red[g][c] = t;
  __syncthreads();
  if (g == 0 && n < N) {
    float r = accumulate ? out[n] : 0.f;
    r += red[0][c];
    r += red[1][c];
    r += red[2][c];
    r += red[3][c];
    out[n] = r;
  }
}

}  // namespace

hipError_t launch_shard_reduce(const float* const* parts, int k, float* Z, int64_t n,
                               hipStream_t s) {
  PartPtrs pp;
  for (int i = 0; i < 64; ++i) pp.p[i] = i < k ? parts[i] : nullptr;
  return launch_reduce_u<4>(pp, k, Z, n, 65536, s);
}

int64_t colsum_partials_floats(int64_t M, int64_t N) { return colsum_row_blocks(M, N) * N; }

hipError_t launch_colsum(const void* const* A, int groups, bool bf16, int64_t M, int64_t N,
                         float* const* out, bool accumulate, float* partials, hipStream_t s) {
  if (N <= 0 || groups < 1) return hipSuccess;
  if (groups > kMaxGroups) return hipErrorInvalidValue;
  ColsumPtrs pp{};
  for (int g = 0; g < groups; ++g) {
    pp.A[g] = A[g];
    pp.out[g] = out[g];
  }
  const int64_t rb = colsum_row_blocks(M, N);
  if (rb > 0) {
    const int64_t rows = (M + rb - 1) / rb;
    const dim3 grid((unsigned)((N + kColsPerBlock - 1) / kColsPerBlock), (unsigned)rb, (unsigned)groups);
    if (bf16)
      hipLaunchKernelGGL(colsum_partial_kernel<true>, grid, dim3(256), 0, s, pp, M, N, rows, partials);
    else
      hipLaunchKernelGGL(colsum_partial_kernel<false>, grid, dim3(256), 0, s, pp, M, N, rows, partials);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((N + 63) / 64), (unsigned)groups), dim3(256), 0,
                     s, pp, partials, rb, N, accumulate ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K-split sums: C[g] = C[g] + part[g (n - 1)] + ... + part[g (n - 1) + n - 2]
// for every group g, in slice order, one launch (blockIdx.y = group).
// ---------------------------------------------------------------------------
struct SplitPtrs {
  float* C[kMaxGroups];
};

template <int NC>
__global__ __launch_bounds__(256) void split_reduce_kernel(SplitPtrs pp, const float* __restrict__ part,
                                                           int64_t part_stride, int n, int64_t count) {
  constexpr int U = 4;
  const int nn = NC > 0 ? NC : n;
  const int g = blockIdx.y;
  float* __restrict__ C = pp.C[g];
  const float* __restrict__ base = part + (int64_t)g * (nn - 1) * part_stride;
  const int64_t n4 = count >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
  for (int64_t v0 = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; v0 < n4; v0 += stride) {
    f32x4_t acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      acc[u] = v < n4 ? reinterpret_cast<const f32x4_t*>(C)[v] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (NC > 0) {
      f32x4_t t[NC > 1 ? NC - 1 : 1][U];
#pragma unroll
      for (int i = 1; i < NC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          t[i - 1][u] = v < n4 ? __builtin_nontemporal_load(
                                     reinterpret_cast<const f32x4_t*>(base + (i - 1) * part_stride) + v)
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int i = 1; i < NC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = acc[u] + t[i - 1][u];
    } else {
      for (int i = 1; i < nn; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          if (v < n4)
            acc[u] = acc[u] + __builtin_nontemporal_load(
                                  reinterpret_cast<const f32x4_t*>(base + (i - 1) * part_stride) + v);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      if (v < n4) reinterpret_cast<f32x4_t*>(C)[v] = acc[u];
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (count & 3)) {
    const int64_t e = (n4 << 2) + threadIdx.x;
    float t = C[e];
    for (int i = 1; i < nn; ++i) t = t + base[(i - 1) * part_stride + e];
    C[e] = t;
  }
}

hipError_t launch_split_reduce(float* const* C, int groups, const float* part, int64_t part_stride,
                               int n, int64_t count, hipStream_t s) {
  if (n <= 1 || count <= 0 || groups < 1) return hipSuccess;
  if (groups > kMaxGroups) return hipErrorInvalidValue;
  SplitPtrs pp{};
  for (int g = 0; g < groups; ++g) pp.C[g] = C[g];
  int64_t blocks = ((count >> 2) + 1023) / 1024;
  const int64_t cap = 2048 / groups + 1;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)groups), block(256);
  switch (n) {
    case 2: hipLaunchKernelGGL(split_reduce_kernel<2>, grid, block, 0, s, pp, part, part_stride, n, count); break;
    case 4: hipLaunchKernelGGL(split_reduce_kernel<4>, grid, block, 0, s, pp, part, part_stride, n, count); break;
    case 8: hipLaunchKernelGGL(split_reduce_kernel<8>, grid, block, 0, s, pp, part, part_stride, n, count); break;
    default: hipLaunchKernelGGL(split_reduce_kernel<0>, grid, block, 0, s, pp, part, part_stride, n, count); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sequence-parallel reduce-scatter with the residual: rank r = blockIdx.y
// owns rows [r Mb, (r + 1) Mb), i.e. the block_elems = Mb H contiguous floats
// at r block_elems of every part, and writes
//   O_r[e] = R[r block_elems + e] + ((P_0 + P_1) + ... + P_{n-1})[r block_elems + e]
// in float32 (R == nullptr: no residual), rounded to nearest-even bf16 when
// OBF16.  block_elems is a multiple of 8, so every 16-byte vector of a part
// lies in one rank's block.
// ---------------------------------------------------------------------------
struct SpPtrs {
  const float* p[64];
  void* out[64];
};

template <int KC, bool RBF16, bool OBF16>
__global__ __launch_bounds__(256) void sp_reduce_kernel(SpPtrs pp, int nparts, const void* __restrict__ R,
                                                        int64_t block_elems) {
  constexpr int U = 4;
  const int kk = KC > 0 ? KC : nparts;
  const int64_t n4 = block_elems >> 2;
  const int64_t base4 = (int64_t)blockIdx.y * n4;  // this rank's first vector in a part
  void* __restrict__ out = pp.out[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
  const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int64_t v0 = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; v0 < n4; v0 += stride) {
    f32x4_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      s[u] = v < n4 ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pp.p[0]) + base4 + v)
                    : zero;
    }
    if constexpr (KC > 0) {
      f32x4_t t[KC > 1 ? KC - 1 : 1][U];
#pragma unroll
      for (int i = 1; i < KC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          t[i - 1][u] = v < n4 ? __builtin_nontemporal_load(
                                     reinterpret_cast<const f32x4_t*>(pp.p[i]) + base4 + v)
                               : zero;
        }
#pragma unroll
      for (int i = 1; i < KC; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = s[u] + t[i - 1][u];
    } else {
      for (int i = 1; i < kk; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t v = v0 + (int64_t)u * blockDim.x;
          if (v < n4)
            s[u] = s[u] + __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pp.p[i]) + base4 + v);
        }
    }
    if (R) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + (int64_t)u * blockDim.x;
        if (v >= n4) continue;
        f32x4_t r;
        if constexpr (RBF16) {
          const u32x2_t h = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(R) + base4 + v);
          r = f32x4_t{bf16_bits_to_f32(h[0] & 0xFFFFu), bf16_bits_to_f32(h[0] >> 16),
                      bf16_bits_to_f32(h[1] & 0xFFFFu), bf16_bits_to_f32(h[1] >> 16)};
        } else {
          r = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(R) + base4 + v);
        }
        s[u] = r + s[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t v = v0 + (int64_t)u * blockDim.x;
      if (v >= n4) continue;
      if constexpr (OBF16) {
        const u32x2_t o = u32x2_t{f32_to_bf16_bits(s[u][0]) | (f32_to_bf16_bits(s[u][1]) << 16),
                                  f32_to_bf16_bits(s[u][2]) | (f32_to_bf16_bits(s[u][3]) << 16)};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(out) + v);
      } else {
        __builtin_nontemporal_store(s[u], reinterpret_cast<f32x4_t*>(out) + v);
      }
    }
  }
}

template <bool RBF16, bool OBF16>
void launch_sp_typed(const SpPtrs& pp, int nparts, const void* R, int k, int64_t block_elems,
                     hipStream_t s) {
  int64_t blocks = ((block_elems >> 2) + 1023) / 1024;
  const int64_t cap = 4096 / k + 1;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks, (unsigned)k), block(256);
  switch (nparts) {
    case 1: hipLaunchKernelGGL((sp_reduce_kernel<1, RBF16, OBF16>), grid, block, 0, s, pp, nparts, R, block_elems); break;
    case 2: hipLaunchKernelGGL((sp_reduce_kernel<2, RBF16, OBF16>), grid, block, 0, s, pp, nparts, R, block_elems); break;
    case 4: hipLaunchKernelGGL((sp_reduce_kernel<4, RBF16, OBF16>), grid, block, 0, s, pp, nparts, R, block_elems); break;
    case 8: hipLaunchKernelGGL((sp_reduce_kernel<8, RBF16, OBF16>), grid, block, 0, s, pp, nparts, R, block_elems); break;
    default: hipLaunchKernelGGL((sp_reduce_kernel<0, RBF16, OBF16>), grid, block, 0, s, pp, nparts, R, block_elems); break;
  }
}

hipError_t launch_sp_reduce_scatter(const float* const* parts, int nparts, const void* R, bool r_bf16,
                                    void* const* out, bool o_bf16, int k, int64_t block_elems,
                                    hipStream_t s) {
  if (nparts < 1 || nparts > 64 || k < 1 || k > 64 || block_elems % 8) return hipErrorInvalidValue;
  if (block_elems == 0) return hipSuccess;
  SpPtrs pp{};
  for (int i = 0; i < nparts; ++i) pp.p[i] = parts[i];
  for (int r = 0; r < k; ++r) pp.out[r] = out[r];
  if (r_bf16) {
    if (o_bf16) launch_sp_typed<true, true>(pp, nparts, R, k, block_elems, s);
    else launch_sp_typed<true, false>(pp, nparts, R, k, block_elems, s);
  } else {
    if (o_bf16) launch_sp_typed<false, true>(pp, nparts, R, k, block_elems, s);
    else launch_sp_typed<false, false>(pp, nparts, R, k, block_elems, s);
  }
  return hipGetLastError();
}

}  // namespace tpmlp
