// float32 GEMM for gfx950: C[M,N] = epilogue(A B) with float32 operands on
// v_mfma_f32_16x16x4_f32, for the operand layouts kNN, kNT and kTN.
//
// 64 x 64 workgroup tile, K step 16, 4 waves of 32 x 32, each a 2 x 2 block
// of 16x16 MFMA tiles.  LDS holds A as [k][m] and B as [k][n] whatever their
// layout in memory (a K-major operand is transposed on its way into LDS), so
// both MFMA operands are read as consecutive words across lanes.  This is the
// full-precision path; the bf16 kernels carry the throughput.
//
// kEpiSwiGLU (kNN only) multiplies A by two B operands, B and B2, in the same
// K loop (a second B tile in LDS and a second accumulator set) and stores
// SiLU(A B) * (A B2).
#include <type_traits>
#include <utility>

#include "device_common.h"
#include "tp_mlp_kernels.h"

namespace tpmlp {

namespace {

struct F32Params {
  const float* A;
  const float* B;
  const float* B2;  // kEpiSwiGLU
  const float* bias;
  float* C;
  float* aux;
  int64_t lda, ldb, ldc;
  int64_t M;
  int N, K;
  int tiles_m, tiles_n;
};

template <int EPI, int LAYOUT>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  constexpr int BM = 64, BN = 64, BK = 16, PAD = 4;
  constexpr bool AK = LAYOUT != kTN;  // A K-major
  constexpr bool BKM = LAYOUT == kNT; // B K-major
  constexpr bool DUAL = EPI == kEpiSwiGLU;
  static_assert(!DUAL || LAYOUT == kNN, "SwiGLU: kNN");
  __shared__ __attribute__((aligned(16))) float As[BK][BM + PAD];
  __shared__ __attribute__((aligned(16))) float Bs[BK][BN + PAD];
  __shared__ __attribute__((aligned(16))) float Bs2[DUAL ? BK : 1][BN + PAD];

  int tm, tn;
  tile_coords<8>(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, tm, tn);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t M = p.M;
  const int N = p.N, K = p.K;

  f32x4_t acc[2][2], acc2[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = acc2[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A K-major / B K-major: thread loads 4 consecutive k of row (tid / 4).
  // A M-major / B N-major: thread loads 4 consecutive m (n) of k-row (tid / 16).
  const int kr = tid >> 2, kc = (tid & 3) * 4;
  const int xr = tid >> 4, xc = (tid & 15) * 4;
  const f32x4_t zero = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += BK) {
    f32x4_t va = zero, vb = zero, vb2 = zero;
    if constexpr (AK) {
      if (m0 + kr < M && k0 + kc < K)
        va = *reinterpret_cast<const f32x4_t*>(p.A + (m0 + kr) * p.lda + k0 + kc);
    } else {
      if (k0 + xr < K && m0 + xc < M)
        va = *reinterpret_cast<const f32x4_t*>(p.A + (int64_t)(k0 + xr) * p.lda + m0 + xc);
    }
    if constexpr (BKM) {
      if (n0 + kr < N && k0 + kc < K)
        vb = *reinterpret_cast<const f32x4_t*>(p.B + (n0 + kr) * p.ldb + k0 + kc);
    } else {
      if (k0 + xr < K && n0 + xc < N) {
        vb = *reinterpret_cast<const f32x4_t*>(p.B + (int64_t)(k0 + xr) * p.ldb + n0 + xc);
        if constexpr (DUAL)
          vb2 = *reinterpret_cast<const f32x4_t*>(p.B2 + (int64_t)(k0 + xr) * p.ldb + n0 + xc);
      }
    }
    if constexpr (AK) {
#pragma unroll
      for (int j = 0; j < 4; ++j) As[kc + j][kr] = va[j];
    } else {
      *reinterpret_cast<f32x4_t*>(&As[xr][xc]) = va;
    }
    if constexpr (BKM) {
#pragma unroll
      for (int j = 0; j < 4; ++j) Bs[kc + j][kr] = vb[j];
    } else {
      *reinterpret_cast<f32x4_t*>(&Bs[xr][xc]) = vb;
      if constexpr (DUAL) *reinterpret_cast<f32x4_t*>(&Bs2[xr][xc]) = vb2;
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < BK / 4; ++kq) {
      const int kk = kq * 4 + (lane >> 4);
      float a_op[2], b_op[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) a_op[j] = Bs[kk][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i) b_op[i] = As[kk][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_op[j], b_op[i], acc[i][j], 0, 0, 0);
      if constexpr (DUAL) {
        float a2_op[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) a2_op[j] = Bs2[kk][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc2[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2_op[j], b_op[i], acc2[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 32 + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 32 + j * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      const int64_t idx = m * p.ldc + n;
      f32x4_t v = acc[i][j];
      if constexpr (EPI == kEpiBias) {
        if (p.bias) v += *reinterpret_cast<const f32x4_t*>(p.bias + n);
        *reinterpret_cast<f32x4_t*>(p.C + idx) = v;
      } else if constexpr (EPI == kEpiBiasGelu || EPI == kEpiBiasGeluSave) {
        if (p.bias) v += *reinterpret_cast<const f32x4_t*>(p.bias + n);
        f32x4_t y, g;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (EPI == kEpiBiasGelu) {
            y[e] = gelu_f32(v[e]);
          } else {
            float ye, ge;
            gelu_and_grad_f32(v[e], ye, ge);
            y[e] = ye;
            g[e] = ge;
          }
        }
        *reinterpret_cast<f32x4_t*>(p.C + idx) = y;
        if constexpr (EPI == kEpiBiasGeluSave) *reinterpret_cast<f32x4_t*>(p.aux + idx) = g;
      } else if constexpr (DUAL) {
        const f32x4_t u = acc2[i][j];
        f32x4_t y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = silu_f32(v[e]) * u[e];
        *reinterpret_cast<f32x4_t*>(p.C + idx) = y;
      } else if constexpr (EPI == kEpiMulAux) {
        const f32x4_t gg = *reinterpret_cast<const f32x4_t*>(p.aux + idx);
        *reinterpret_cast<f32x4_t*>(p.C + idx) = v * gg;
      } else if constexpr (EPI == kEpiStoreF32) {
        *reinterpret_cast<f32x4_t*>(p.C + idx) = v;
      } else {
        f32x4_t* q = reinterpret_cast<f32x4_t*>(p.C + idx);
        const f32x4_t old = *q;
        *q = old + v;
      }
    }
  }
}

template <int LAYOUT>
hipError_t launch_f32_layout(const F32Params& p, Epilogue epi, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  switch (epi) {
    case kEpiBiasGelu:
      hipLaunchKernelGGL((gemm_f32_kernel<kEpiBiasGelu, LAYOUT>), grid, block, 0, s, p);
      break;
    case kEpiStoreF32:
      hipLaunchKernelGGL((gemm_f32_kernel<kEpiStoreF32, LAYOUT>), grid, block, 0, s, p);
      break;
    case kEpiAccumF32:
      hipLaunchKernelGGL((gemm_f32_kernel<kEpiAccumF32, LAYOUT>), grid, block, 0, s, p);
      break;
    case kEpiBiasGeluSave:
      hipLaunchKernelGGL((gemm_f32_kernel<kEpiBiasGeluSave, LAYOUT>), grid, block, 0, s, p);
      break;
    case kEpiMulAux:
      hipLaunchKernelGGL((gemm_f32_kernel<kEpiMulAux, LAYOUT>), grid, block, 0, s, p);
      break;
    case kEpiBias:
      if constexpr (LAYOUT == kNN) {
        hipLaunchKernelGGL((gemm_f32_kernel<kEpiBias, kNN>), grid, block, 0, s, p);
        break;
      }
      return hipErrorInvalidValue;
    case kEpiSwiGLU:
      if constexpr (LAYOUT == kNN) {
        hipLaunchKernelGGL((gemm_f32_kernel<kEpiSwiGLU, kNN>), grid, block, 0, s, p);
        break;
      }
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

constexpr int64_t kMaxTilesPerLaunch = int64_t(1) << 22;

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const int64_t tiles_n = (g.N + 63) / 64;
  const int64_t rows_per_launch = (kMaxTilesPerLaunch / tiles_n) * 64;
  const bool a_kmajor = g.layout != kTN;
  const float* A = static_cast<const float*>(g.A);
  F32Params p;
  p.B = static_cast<const float*>(g.B);
  p.B2 = static_cast<const float*>(g.B2);
  p.bias = static_cast<const float*>(g.bias);
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.ldc = g.ldc;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.tiles_n = (int)tiles_n;
  for (int64_t r0 = 0; r0 < g.M; r0 += rows_per_launch) {
    const int64_t Mc = g.M - r0 < rows_per_launch ? g.M - r0 : rows_per_launch;
    p.A = a_kmajor ? A + r0 * g.lda : A + r0;
    p.C = static_cast<float*>(g.C) + r0 * g.ldc;
    p.aux = g.aux ? static_cast<float*>(g.aux) + r0 * g.ldc : nullptr;
    p.M = Mc;
    p.tiles_m = (int)((Mc + 63) / 64);
    const dim3 grid((unsigned)(p.tiles_m * tiles_n));
    hipError_t e;
    switch (g.layout) {
      case kNN: e = launch_f32_layout<kNN>(p, g.epi, grid, s); break;
      case kNT: e = launch_f32_layout<kNT>(p, g.epi, grid, s); break;
      default: e = launch_f32_layout<kTN>(p, g.epi, grid, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_f32_batch(const GemmBatch& b, hipStream_t s) {
  for (int g = 0; g < b.groups; ++g) {
    GemmArgs a{b.A[g], b.B[g], b.bias[g], b.B2[g], b.group_sum ? b.C[0] : b.C[g], b.aux[g], b.M, b.N, b.K,
               b.lda, b.ldb, b.ldc, b.layout, b.epi};
    if (b.group_sum && g > 0) a.epi = kEpiAccumF32;  // C[0] += A[g] B[g], in group order
    const hipError_t e = launch_gemm_f32(a, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tpmlp
